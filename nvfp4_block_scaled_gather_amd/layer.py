"""Device-side setup of one MoE layer for a workload: packed expert weights resident in
HBM, per-expert globals, routing inputs and the layer workspace.  All compute goes
through the C ABI (``binding``); torch only allocates device memory.
"""
import concurrent.futures

import numpy as np

from . import binding as B


def _dev(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def pack_expert_weights(weight_fn, E, N, K, device="cuda", experts=None):
    """Pack E experts' canonical NVFP4 weights ``weight_fn(e) -> (nib, scl)`` into one
    device buffer, expert by expert (host generation of the next expert overlaps the
    upload and packing of the current one).  Experts not in ``experts`` are left zero."""
    import torch
    per = B.nvfp4_packed_weight_bytes(1, N, K)
    if per == 0:
        raise ValueError("unsupported weight shape N=%d K=%d" % (N, K))
    packed = torch.zeros(per * E, dtype=torch.uint8, device=device)
    todo = list(range(E)) if experts is None else sorted(set(experts))
    nib_d = torch.empty((N, K // 2), dtype=torch.uint8, device=device)
    scl_d = torch.empty((N, K // 16), dtype=torch.uint8, device=device)
    with concurrent.futures.ThreadPoolExecutor(4) as ex:
        futs = [ex.submit(weight_fn, e) for e in todo]
        for e, f in zip(todo, futs):
            nib, scl = f.result()
            nib_d.copy_(torch.from_numpy(nib))
            scl_d.copy_(torch.from_numpy(scl))
            B.nvfp4_pack_weights(nib_d, scl_d, 1, N, K, packed[e * per:(e + 1) * per])
    torch.cuda.synchronize()
    return packed


class DeviceLayer:
    """One layer's resident weights and descriptor for a ``workloads.Workload``."""

    def __init__(self, wl, device="cuda", flags=B.MOE_PATH_AUTO,
                 gemv_max_rows=B.DEFAULT_GEMV_MAX_ROWS, experts=None, weights=None,
                 arithmetic="w4a4"):
        """``weights``: already packed (w13, w2) device buffers of the same expert set
        (workloads of one weight seed share them); otherwise they are packed here.
        ``arithmetic``: "w4a4" (moe_layer_forward: NVFP4 activations) or "w4a16"
        (moe_layer_forward_w4a16: bf16 activations against the same weights)."""
        import torch
        if arithmetic not in ("w4a4", "w4a16"):
            raise ValueError("arithmetic must be 'w4a4' or 'w4a16', got %r" % (arithmetic,))
        self.arithmetic = arithmetic
        self.wl = wl
        self.device = device
        if weights is None:
            weights = (pack_expert_weights(wl.w13, wl.E, 2 * wl.I, wl.H, device, experts),
                       pack_expert_weights(wl.w2, wl.E, wl.H, wl.I, device, experts))
        self.w13, self.w2 = weights
        self.g_gate = _dev(wl.g_gate, device)
        self.g_up = _dev(wl.g_up, device)
        self.g_down = _dev(wl.g_down, device)
        self.set_path(flags, gemv_max_rows)
        self.x = _dev(wl.x.view(np.int16), device)
        self.a_expert = _dev(wl.a_expert, device)
        self.a_src = _dev(wl.a_src, device)
        self.a_dst = _dev(wl.a_dst, device)
        self.a_w = _dev(wl.a_w, device)
        self.ws_bytes = B.moe_layer_workspace_bytes(self.desc, wl.S, wl.R, wl.T)
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        # 256-byte aligned view
        off = (-self.ws.data_ptr()) % 256
        self.ws_view = self.ws[off:off + self.ws_bytes]
        self.out = torch.empty((wl.T, wl.H), dtype=torch.int16, device=device)

    def set_path(self, flags, gemv_max_rows):
        wl = self.wl
        self.desc = B.make_layer_desc(wl.E, wl.H, wl.I, self.w13, self.w2, self.g_gate, self.g_up,
                                      self.g_down, flags, gemv_max_rows)

    def forward(self, stream=None):
        wl = self.wl
        fn = B.moe_layer_forward if self.arithmetic == "w4a4" else B.moe_layer_forward_w4a16
        fn(self.desc, self.x, wl.S, self.a_expert, self.a_src, self.a_dst, self.a_w, wl.R, wl.T,
           self.out, self.ws_view, self.ws_bytes, stream)
        return self.out

    def device_error(self):
        return B.moe_get_device_error(self.ws_view)

    def capture_graph(self):
        """A HIP graph of one forward() (its kernel launches, no memset nodes); replaying
        it recomputes self.out from the resident inputs.  Warmed up eagerly on the capture
        stream first."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                self.forward()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward()
        torch.cuda.synchronize()
        return graph

    def weight_stream_bytes(self):
        """Weight bytes one layer call streams: active experts x (w13 + w2) packed bytes,
        the byte model of the page's table "Bytes decide it before the kernel runs"."""
        wl = self.wl
        return weight_stream_bytes(len(wl.active_experts()), wl.H, wl.I)


def weight_stream_bytes(n_active, H, I):
    """n_active * (2I*H + H*I) * (0.5 + 1/16) bytes."""
    return n_active * (2 * I * H + H * I) * 9 // 16
