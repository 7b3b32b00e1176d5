"""MoE expert-FFN layer hot path for MI355X (gfx950): router top-k, device-resident routing
metadata, rowwise permute, device-scheduled grouped GEMM SwiGLU experts in bf16 and MXFP8,
weighted unpermute-combine, and the backward, as hand-written HIP kernels behind a C ABI
(include/moe_mi355x.h).

  ops    thin torch wrappers of every C entry point (marshalling only)
  layer  the whole layer step (forward + backward) composed from those entry points
  build  compiles csrc/*.hip into libmoe_mi355x.so in-tree
"""

__all__ = ["ops", "layer"]


def __getattr__(name):
    # the HIP library is loaded on first use of ops/layer, so `build` works without it
    if name in ("ops", "layer"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
