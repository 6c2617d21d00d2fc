"""MI355X-native MoE expert-layer forward: route -> permute -> grouped GEMM
(gate/up + SwiGLU, down) -> combine, as hand-written HIP kernels for gfx950
behind the C-ABI library ``libmoe.so`` (declared in ``include/moe.h``).

Importing the package does not load the library; ``grouped_gemm_router_amd.api``
does, and raises if it is missing.  ``synth`` holds the seeded input
generators and workload shapes.
"""
__all__ = ["api", "layer", "synth"]
