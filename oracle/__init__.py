"""CPU oracle for the NVFP4 routed-expert MoE layer path — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct numpy implementation of every step of
the path.  It exists to check the HIP library; it is not part of the product.  Only the
test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import it.  It imports nothing from the HIP package and shares no code with it.

Sources (cited by page title and section; the pages are the authority):

* [GG] "The CUTLASS grouped GEMM beats the scalar GEMV loop at every M, M=1 included,
  so the crossover is 1" (gabewillen.github.io/rocket, posts/runtime, 2026-09-07).
  Section "What changed" lists the seven steps of the routed-expert loop; section
  "The seam CUTLASS forced open" fixes the fused gate|up operand; section "Proof"
  lists the invariants (row invariance, fused == separate, determinism) and the
  kernel checks.
* [MF] "Fusing the MoE layer's two grouped GEMMs is worth 4%, and a CUDA graph
  already collects it" (gabewillen.github.io/rocket, posts/kernels, 2026-09-06).
  Table "Bytes decide it before the kernel runs" gives the NVFP4 byte model;
  section "Different globals on the two halves" fixes where the gate/up globals
  apply (option (a)) and the e4m3 fold-probe statistics.

Arithmetic: float64 everywhere except the quantizer, which the plainest NVFP4 reading
defines in float32 (see ``nvfp4.quantize_row``).

Parity status of each function is stated in its docstring.  The end-to-end layer
(``moe.layer_forward``) is pinned only through the composition of its pinned steps
plus invariants; beyond that composition, END-TO-END PARITY IS UNPINNED.
"""
from . import nvfp4, moe  # noqa: F401
