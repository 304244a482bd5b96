"""CPU oracle for one forward pass of the Stable LatentMoE layer with MXFP4 routed experts.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
never imports the product path.  The two share only the seeded input
generators in `synth`, which hold none of the layer's arithmetic.

The oracle is the plain definition of the layer written out in float64 numpy
(library matmuls for the dense products), with one exception fixed by the
method's statement of the router: the top-k *decision* is taken on float32
biased scores.  Every function names the passage of the pages it follows:

  * kimi-k3-mlx README (PipeNetwork/kimi-k3-mlx): Architecture table (MoE,
    Stable LatentMoE, Activation and Source-format rows), Porting notes item 1
    (SiTU-GLU in fp32) and item 3 (experts in the latent, shared experts not),
    Tiers section (mxfp4: low-nibble-first e2m1 codes, e8m0 scales), REAP
    section (pairs sorted by expert index give contiguous slices; RMSNorm acts
    on the combined expert output), AWQ section (one latent feeds every
    expert).
  * K3 open-artifact audit (llm-atlas), section 4.3 (the MXFP4 tensors of one
    routed expert) and section 6 (router weight and fp32 correction bias).

Modules:
  mxfp4   -- e2m1 code table and MXFP4 dequantisation
  layer   -- routing, permutation, expert MLP, combine/RMSNorm/up_proj,
             shared experts, the layer forward, the grouped-GEMM microbench
  scalar  -- a second, structurally different tiny-shape oracle (per-token,
             per-pair Python loops, its own bit-level e2m1 decoding)
  reap    -- REAP expert saliency over a calibration batch (README, REAP
             section)
  promotion -- the moe_k_hi cap on promoted (MXFP4) experts per token
             (Kimi-K3-Alis-MLX-Dynamic card, Build recipe)

Parity status: the whole-layer result has no worked input/output example on
the pages; it is pinned by the independent scalar oracle, by closed forms and
limits (SiTU-GLU), brute force (e2m1 bytes, top-k subsets), invariants
(RMSNorm scale invariance, pruning equivalence, zero codes) and the pages'
printed shape and parameter counts.
"""
from . import mxfp4, layer, scalar, reap  # noqa: F401
