"""CPU oracle for one GPU's share of an expert-parallel MoE layer (router, routing
metadata, rowwise permute, SwiGLU expert FFN, weighted combine, and their backward;
MXFP8 block quantisation).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package: only
the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It is a plain,
slow, obviously-correct restatement of what the layer computes, in numpy float64 (bf16
and fp32 inputs are exact in float64), and it shares no code with the HIP library.

Sources.  The method is the MoE layer of the Olmo-core 3 training stack:
  * "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs" (news page),
    lead paragraphs (a router sends each token to a few FFN experts), section
    "Routing work stays on the GPU" (rows written straight into expert input buffers,
    device-resident routing metadata, grouped GEMM) and section "MXFP8 reduces compute
    and memory costs" (8-bit floats with one scale per small block).
  * "Supercharging Olmo-core for Efficient and Scalable MoE Training" (paper card),
    section "Summary" (rowwise EP, GPU-resident routing metadata, device-scheduled
    grouped GEMMs, MXFP8).
The pages name these steps but give no arithmetic.  The arithmetic (softmax over all
experts, top-k with renormalised gates, SwiGLU experts, E4M3 elements with one E8M0
scale per 32 elements along the contraction dimension, bf16 storage with fp32
accumulation) is the layer specification this library implements; every reading made
where it is silent is listed in the design notes of the repository.

Modules
  codecs   bf16 / E4M3 / E8M0 bit codecs
  moe      the layer's steps, forward and backward, one function per library entry point
  moe_mx   the layer with every expert product on MXFP8 operands, as a chain of those steps
  mxfp8    MX block quantisation (row blocks, column blocks, grouped token blocks)
  sampled  per-row / per-expert evaluators for checking full-size runs on samples

Every function here is pinned in tests/test_oracle_*.py against something other than
itself (brute force, closed forms, invariants, CPU torch, exhaustive enumeration).
"""

from . import codecs, moe, moe_mx, mxfp8, sampled  # noqa: F401
