"""Routed-expert MoE layer steps (CPU oracle; test infrastructure only).

The layer is the routed-expert loop of [GG] section "What changed":
  gather -> quantize -> grouped GEMM (w13, fused gate|up) -> SwiGLU (per-half globals)
  -> quantize -> grouped GEMM (w2) -> scatter-add weighted by router weight * down global.
Each function below is one of those steps, in float64 unless stated otherwise.  The W4A16
variant (grouped_gemm_w4a16, layer_forward_w4a16) is the same loop without the two
activation quantizations: bf16 activations against the NVFP4 weights, the arithmetic of
the pages' dequant-GEMV path ([GG] "Numbers").

Notation: E experts, H hidden, I intermediate, S activation source rows, T output rows
(tokens), R assignments ("expert-rows").  An assignment j routes source row a_src[j] to
expert a_expert[j]; its result lands in output row a_dst[j] with router weight a_w[j].

Weights are canonical NVFP4 per expert: nibbles [N, K/2] (even element in the low
nibble) and e4m3 scales [N, K/16].  w13 has N = 2I rows: rows [0, I) are the gate
projection and rows [I, 2I) the up projection ([GG] "The seam CUTLASS forced open": the
gate matrix followed by the up matrix is itself the fused w13 operand).  w2 has N = H rows
and K = I.
"""
import numpy as np

from . import nvfp4

ERR_EXPERT = 1   # a_expert[j] outside [0, E)
ERR_SRC = 2      # a_src[j] outside [0, S)
ERR_DST = 4      # a_dst[j] outside [0, T)


def group_rows(a_expert, a_src, a_dst, a_w, E, S, T):
    """Group assignments by expert id, ascending ([GG] "What changed": the batch's rows are
    collected per expert in an ordered map, so the groups come out in ascending expert id
    and their order depends on nothing but the set of experts that received rows).  Within
    an expert, rows keep their assignment order.

    Assignments with an out-of-range expert, source or destination are dropped; their
    error bits are OR-ed into ``err``.  Dropped rows occupy the tail i >= offsets[E]
    with row_src = row_dst = -1 and row_w = 0, in ascending assignment order.

    Returns dict: offsets [E+1], row_expert, row_src, row_dst, row_w [R],
    tok_off [T+1], tok_rows [offsets[E]], err (int).
    """
    a_expert = np.asarray(a_expert, dtype=np.int64)
    a_src = np.asarray(a_src, dtype=np.int64)
    a_dst = np.asarray(a_dst, dtype=np.int64)
    a_w = np.asarray(a_w, dtype=np.float32)
    R = len(a_expert)
    err = 0
    valid = []
    for j in range(R):
        bad = 0
        if not (0 <= a_expert[j] < E):
            bad |= ERR_EXPERT
        if not (0 <= a_src[j] < S):
            bad |= ERR_SRC
        if not (0 <= a_dst[j] < T):
            bad |= ERR_DST
        err |= bad
        valid.append(bad == 0)
    good = [j for j in range(R) if valid[j]]
    dropped = [j for j in range(R) if not valid[j]]
    order = sorted(good, key=lambda j: (a_expert[j], j))
    Rv = len(order)
    offsets = np.zeros(E + 1, dtype=np.int32)
    for j in order:
        offsets[a_expert[j] + 1] += 1
    offsets = np.cumsum(offsets).astype(np.int32)
    row_expert = np.full(R, E, dtype=np.int32)
    row_src = np.full(R, -1, dtype=np.int32)
    row_dst = np.full(R, -1, dtype=np.int32)
    row_w = np.zeros(R, dtype=np.float32)
    for i, j in enumerate(order):
        row_expert[i] = a_expert[j]
        row_src[i] = a_src[j]
        row_dst[i] = a_dst[j]
        row_w[i] = a_w[j]
    del dropped  # their slots keep the sentinel values above
    # token CSR: for each output row t, the grouped rows i that land in it, ascending i
    tok_lists = [[] for _ in range(T)]
    for i in range(Rv):
        tok_lists[row_dst[i]].append(i)
    tok_off = np.zeros(T + 1, dtype=np.int32)
    for t in range(T):
        tok_off[t + 1] = tok_off[t] + len(tok_lists[t])
    tok_rows = np.array([i for t in range(T) for i in tok_lists[t]], dtype=np.int32)
    return dict(offsets=offsets, row_expert=row_expert, row_src=row_src, row_dst=row_dst,
                row_w=row_w, tok_off=tok_off, tok_rows=tok_rows, err=err)


def gather_rows(x_bits, row_src):
    """xg[i] = x[row_src[i]] ([GG] "What changed": one row per (stream, expert)); rows
    with row_src < 0 (dropped) are zero.  Works on raw bf16 bit patterns: exact copy."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    out = np.zeros((len(row_src), x_bits.shape[1]), dtype=np.uint16)
    for i, s in enumerate(row_src):
        if s >= 0:
            out[i] = x_bits[s]
    return out


def grouped_gemm(aq, as_, offsets, weights, N, K):
    """acc[i, n] = sum_k a(i, k) * w_e(n, k) for every row i of expert e's group, in float64.

    a and w are the exact NVFP4 values e2m1 * e4m3 (no globals: the GEMM runs with
    alpha = 1, [GG] "What changed").  ``weights(e)`` returns expert e's (nibbles, scales).
    Rows outside every group (i >= offsets[E]) are left at zero.
    """
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    R = aq.shape[0]
    acc = np.zeros((R, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue                                  # empty expert: no work
        w_nib, w_sc = weights(e)
        assert w_nib.shape == (N, K // 2) and w_sc.shape == (N, K // 16)
        wd = nvfp4.dequantize(w_nib, w_sc)                # [N, K]
        for i in range(r0, r1):                           # one matrix-vector product per
            xa = nvfp4.dequantize(aq[i], as_[i])          # row, so a row's result cannot
            acc[i] = wd @ xa                              # depend on its group's other rows
    return acc


def grouped_gemm_w4a16(a_bits, offsets, weights, N, K):
    """W4A16: acc[i, n] = sum_k x(i, k) * w_e(n, k) for every row i of expert e's group, in
    float64, with x the row's bf16 values taken exactly (no activation quantization) and w
    the exact NVFP4 weight values.  This is the arithmetic of the pages' dequant-GEMV loop
    ([GG] "Numbers": exact BF16 activations against an NVFP4 weight).  ``a_bits``: bf16 bit
    patterns [R, K]; rows outside every group are left at zero.
    """
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    a = nvfp4.bf16_bits_to_f32(np.asarray(a_bits, dtype=np.uint16)).astype(np.float64)
    R = a.shape[0]
    acc = np.zeros((R, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        w_nib, w_sc = weights(e)
        assert w_nib.shape == (N, K // 2) and w_sc.shape == (N, K // 16)
        wd = nvfp4.dequantize(w_nib, w_sc)
        for i in range(r0, r1):
            acc[i] = wd @ a[i]
    return acc


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(acc13, offsets, g_gate, g_up, row_gs, I):
    """h[i, j] = bf16( silu(z_gate) * z_up ) with, for row i of expert e,
       z_gate = gs_i * g_gate[e] * acc13[i, j],   z_up = gs_i * g_up[e] * acc13[i, I + j].

    The gate and up halves carry their own weight_scale_2 globals, applied here in the
    activation kernel ([MF] "Different globals on the two halves", option (a)); gs_i is
    the row's activation global.  Returns bf16 bit patterns [R, I]; rows outside every
    group are zero.
    """
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    R = acc13.shape[0]
    h = np.zeros((R, I), dtype=np.uint16)
    for e in range(E):
        for i in range(int(offsets[e]), int(offsets[e + 1])):
            gs = np.float64(row_gs[i])
            zg = gs * np.float64(g_gate[e]) * acc13[i, :I]
            zu = gs * np.float64(g_up[e]) * acc13[i, I:2 * I]
            h[i] = nvfp4.f64_to_bf16_bits(silu(zg) * zu)
    return h


def scatter_add(y, offsets, row_w, g_down, row_gs, tok_off, tok_rows, T):
    """out[t] = bf16( sum over grouped rows i of token t, ascending i, of
                       row_w[i] * g_down[e_i] * gs_h[i] * y[i] ).

    Weighted by router weight times the down projection's global ([GG] "What changed"),
    times the row global of the down GEMM's quantized input; accumulation in a shared
    per-token row in order of i ([GG] "Proof", kernel checks).  A token with no rows
    outputs zeros.  Returns bf16 bit patterns [T, H].
    """
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    row_e = np.zeros(len(row_w), dtype=np.int64)
    for e in range(E):
        row_e[int(offsets[e]):int(offsets[e + 1])] = e
    H = y.shape[1]
    out = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for p in range(int(tok_off[t]), int(tok_off[t + 1])):
            i = int(tok_rows[p])
            c = np.float64(row_w[i]) * np.float64(g_down[row_e[i]]) * np.float64(row_gs[i])
            out[t] += c * y[i]
    return nvfp4.f64_to_bf16_bits(out)


def layer_forward(x_bits, a_expert, a_src, a_dst, a_w, T, w13, w2, g_gate, g_up, g_down,
                  E, H, I, return_intermediates=False):
    """The whole routed-expert layer ([GG] "What changed", all seven steps).

    x_bits: bf16 bit patterns [S, H].  w13(e) / w2(e): callables returning expert e's
    canonical (nibbles, scales).  Returns bf16 bits [T, H] (and the intermediates).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    S = x_bits.shape[0]
    g = group_rows(a_expert, a_src, a_dst, a_w, E, S, T)
    Rv = int(g["offsets"][E])
    xg = gather_rows(x_bits, g["row_src"])
    xq, xs, xgs = nvfp4.quantize_rows(nvfp4.bf16_bits_to_f32(xg))
    acc13 = grouped_gemm(xq, xs, g["offsets"], w13, 2 * I, H)
    h = swiglu(acc13, g["offsets"], g_gate, g_up, xgs, I)
    hq, hs, hgs = nvfp4.quantize_rows(nvfp4.bf16_bits_to_f32(h))
    y = grouped_gemm(hq, hs, g["offsets"], w2, H, I)
    out = scatter_add(y, g["offsets"], g["row_w"], g_down, hgs, g["tok_off"], g["tok_rows"], T)
    if return_intermediates:
        return out, dict(group=g, Rv=Rv, xg=xg, xq=xq, xs=xs, xgs=xgs, acc13=acc13, h=h,
                         hq=hq, hs=hs, hgs=hgs, y=y)
    return out


def layer_forward_w4a16(x_bits, a_expert, a_src, a_dst, a_w, T, w13, w2, g_gate, g_up,
                        g_down, E, H, I, return_intermediates=False):
    """The routed-expert layer in W4A16 arithmetic (the same seven steps without the two
    activation quantizations): gathered bf16 rows against the NVFP4 w13, SwiGLU with the
    gate / up globals alone (no activation global: the activations carry none), bf16 h
    against the NVFP4 w2, scatter-add weighted by router weight * down global.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    S = x_bits.shape[0]
    g = group_rows(a_expert, a_src, a_dst, a_w, E, S, T)
    R = len(g["row_src"])
    ones = np.ones(R, dtype=np.float32)
    xg = gather_rows(x_bits, g["row_src"])
    acc13 = grouped_gemm_w4a16(xg, g["offsets"], w13, 2 * I, H)
    h = swiglu(acc13, g["offsets"], g_gate, g_up, ones, I)
    y = grouped_gemm_w4a16(h, g["offsets"], w2, H, I)
    out = scatter_add(y, g["offsets"], g["row_w"], g_down, ones, g["tok_off"], g["tok_rows"], T)
    if return_intermediates:
        return out, dict(group=g, xg=xg, acc13=acc13, h=h, y=y)
    return out
