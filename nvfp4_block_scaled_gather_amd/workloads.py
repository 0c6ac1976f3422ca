"""Seeded synthetic inputs for the MoE layer path (shared by tests, bench and smoke).

This module only draws random inputs.  It contains none of the layer's arithmetic: no
NVFP4 encoding, no quantization, no GEMM.  Both the HIP library and the CPU oracle
consume exactly what it returns.

Workloads (shapes and distributions of the pages' runs, which used a real checkpoint
and real prompts that are not available; these stand in for them):

* ``tiny``:   8 experts, H=256, I=128, 4 tokens, top-2 routing.
* ``decode1``: 288 experts, H=4096, I=2048, 1 token, top-8 (8 groups of one row).
* ``ragged570``: 288 experts, 570 expert-rows, every expert >= 1 row, 8 output rows
  ([MF] "Layer time" / "Tiles below M=8": ragged per-expert M, 570 tokens).
* ``ragged2303``: 288 experts, 2303 expert-rows, 288 output rows of 8 (7 for the last).
* ``zipf512``: 64 tokens, top-8 over 288 experts with Zipf(1.1) popularity.
* ``decode2`` .. ``decode32``: the decode-batch M sweep ([GG] "Numbers", extended past M=8
  as its "Next" list asks): M = 2, 4, 8, 16, 32 token streams, each top-8 over N(0,1)
  logits, as decode1.

Weights for expert e and tensor t come from a counter-based Philox stream keyed by
(weight_seed, e, t), so any expert can be regenerated alone.  The four full-size workloads
share one weight seed (one resident expert set serves all of them); routing and
activations have a seed per workload.
"""
import dataclasses

import numpy as np

G_GATE = np.float32(4.65e-5)   # [MF] "Different globals on the two halves": gate global
G_UP = np.float32(3.78e-5)     # ... and up global (ratio 1.2308)
G_DOWN = np.float32(4.2e-5)

TENSOR_W13 = 0
TENSOR_W2 = 1

WORKLOADS = ("tiny", "decode1", "ragged570", "ragged2303", "zipf512",
             "decode2", "decode4", "decode8", "decode16", "decode32")
DECODE_SWEEP = (1, 2, 4, 8, 16, 32)  # token streams of the decode M-sweep
BASE_SEED = 20260906


def _rng(seed, *key):
    """Counter-based generator keyed by integers (Philox, 2x64-bit key)."""
    k0 = int(seed) & 0xFFFFFFFFFFFFFFFF
    k1 = 0
    for v in key:
        k1 = (k1 * 1000003 + int(v) + 1) & 0xFFFFFFFFFFFFFFFF
    return np.random.Generator(np.random.Philox(key=[k0, k1]))


def expert_weights(seed, e, tensor, N, K):
    """Canonical NVFP4 weights of one expert projection.

    nibbles [N, K/2] uint8: every nibble uniform over all 16 e2m1 codes.
    scales  [N, K/16] uint8: e4m3 block scales, log-uniform in [2^-6, 2^0): draw
      u ~ U(-6, 0), take the binade floor(u) and the mantissa step floor(8*(2^frac - 1)),
      i.e. the e4m3 grid point at or below 2^u.
    """
    g = _rng(seed, 7, e, tensor)
    nib = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    u = g.random((N, K // 16)) * -6.0              # in (-6, 0]
    u = np.where(u == 0.0, -1e-12, u)
    b = np.floor(u)
    frac = np.exp2(u - b)                           # [1, 2)
    m = np.minimum(np.floor((frac - 1.0) * 8.0), 7)
    scl = (((b + 7).astype(np.int64) << 3) | m.astype(np.int64)).astype(np.uint8)
    return nib, scl


def bf16_normal(seed, shape, *key):
    """bf16 bit patterns of N(0,1) samples (rounded to bf16 by torch's own cast)."""
    import torch
    g = _rng(seed, 11, *key)
    f = g.standard_normal(size=shape).astype(np.float32)
    t = torch.from_numpy(f).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _topk_softmax(logits, k):
    """Top-k of each row (ties to the lower index), softmax over the selected logits."""
    T, E = logits.shape
    ids = np.zeros((T, k), dtype=np.int64)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        sel = logits[t, order]
        p = np.exp(sel - sel.max())
        ids[t] = order
        w[t] = p / p.sum()
    return ids, w.astype(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    E: int
    H: int
    I: int
    S: int          # activation source rows
    T: int          # output rows (tokens)
    x: np.ndarray   # bf16 bits [S, H]
    a_expert: np.ndarray  # int32 [R]
    a_src: np.ndarray
    a_dst: np.ndarray
    a_w: np.ndarray       # float32 [R]
    g_gate: np.ndarray    # float32 [E]
    g_up: np.ndarray
    g_down: np.ndarray
    seed: int
    weight_seed: int

    @property
    def R(self):
        return len(self.a_expert)

    def w13(self, e):
        return expert_weights(self.weight_seed, e, TENSOR_W13, 2 * self.I, self.H)

    def w2(self, e):
        return expert_weights(self.weight_seed, e, TENSOR_W2, self.H, self.I)

    def active_experts(self):
        return sorted(set(int(e) for e in self.a_expert if 0 <= e < self.E))


def _topk_workload(name, seed, E, H, I, T, k):
    g = _rng(seed, 1)
    logits = g.standard_normal(size=(T, E))
    ids, w = _topk_softmax(logits, k)
    a_expert = ids.reshape(-1).astype(np.int32)
    a_src = np.repeat(np.arange(T), k).astype(np.int32)
    return a_expert, a_src, a_src.copy(), w.reshape(-1)


def _ragged_counts(g, R, E):
    """Per-expert row counts: 1 + Multinomial(R - E, uniform)."""
    return 1 + g.multinomial(R - E, np.full(E, 1.0 / E))


def make_workload(name, seed=None, E=None, H=None, I=None, weight_seed=None):
    """Build one of the named workloads.  E/H/I override the full dims (tests use
    smaller shapes with the same structure)."""
    idx = WORKLOADS.index(name)
    seed = BASE_SEED + idx if seed is None else seed
    weight_seed = BASE_SEED if weight_seed is None else weight_seed
    full = dict(E=288, H=4096, I=2048)
    if name == "tiny":
        full = dict(E=8, H=256, I=128)
    E = E or full["E"]
    H = H or full["H"]
    I = I or full["I"]
    g = _rng(seed, 2)
    if name == "tiny":
        T = 4
        a_expert, a_src, a_dst, a_w = _topk_workload(name, seed, E, H, I, T, 2)
        S = T
    elif name.startswith("decode"):
        T = int(name[len("decode"):])
        a_expert, a_src, a_dst, a_w = _topk_workload(name, seed, E, H, I, T, min(8, E))
        S = T
    elif name in ("ragged570", "ragged2303"):
        R = 570 if name == "ragged570" else 2303
        R = max(R, E)
        counts = _ragged_counts(g, R, E)
        a_expert = np.repeat(np.arange(E), counts).astype(np.int32)   # ascending expert
        S = R
        a_src = np.arange(R, dtype=np.int32)
        if name == "ragged570":
            T = 8
            a_dst = g.integers(0, T, size=R).astype(np.int32)
            raw = g.random(R)
            a_w = np.zeros(R, dtype=np.float64)
            for t in range(T):
                m = a_dst == t
                if m.any():
                    a_w[m] = raw[m] / raw[m].sum()
            a_w = a_w.astype(np.float32)
        else:
            T = (R + 7) // 8
            perm = g.permutation(R)
            a_dst = np.zeros(R, dtype=np.int32)
            a_dst[perm] = np.arange(R) // 8
            logits = g.standard_normal(R)
            a_w = np.zeros(R, dtype=np.float64)
            for t in range(T):
                m = a_dst == t
                p = np.exp(logits[m] - logits[m].max())
                a_w[m] = p / p.sum()
            a_w = a_w.astype(np.float32)
    elif name == "zipf512":
        T = 64
        k = min(8, E)
        perm = g.permutation(E)
        logp = -1.1 * np.log(perm + 1.0)
        ids = np.zeros((T, k), dtype=np.int64)
        w = np.zeros((T, k), dtype=np.float64)
        for t in range(T):
            pert = logp + g.gumbel(size=E)
            order = sorted(range(E), key=lambda e: (-pert[e], e))[:k]
            sel = pert[order]
            p = np.exp(sel - sel.max())
            ids[t] = order
            w[t] = p / p.sum()
        a_expert = ids.reshape(-1).astype(np.int32)
        a_src = np.repeat(np.arange(T), k).astype(np.int32)
        a_dst = a_src.copy()
        a_w = w.reshape(-1).astype(np.float32)
        S = T
    else:
        raise ValueError(name)
    x = bf16_normal(seed, (S, H), 3)
    return Workload(name=name, E=E, H=H, I=I, S=S, T=T, x=x, a_expert=a_expert,
                    a_src=a_src.astype(np.int32), a_dst=a_dst.astype(np.int32),
                    a_w=a_w.astype(np.float32),
                    g_gate=np.full(E, G_GATE, np.float32), g_up=np.full(E, G_UP, np.float32),
                    g_down=np.full(E, G_DOWN, np.float32), seed=seed, weight_seed=weight_seed)
