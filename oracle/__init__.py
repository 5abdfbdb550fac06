"""CPU oracle for the grouped MoE expert MLP (BF16 and MXFP8, forward and backward).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, smoke() in
__graft_entry__.py and the CPU-baseline leg of bench.py may import, call or
execute anything in this package.  The HIP library never routes through it and
shares no code with it (no kernels, headers, helpers, tables or constants); the
two meet only at the seeded input generator, which holds none of the method's
arithmetic.

The oracle is the plain definition of what the fused path computes: a loop over
experts (the structure of the naive per-expert baseline), torch-CPU matmuls as
the GEMM step, numpy bit operations for the MXFP8 encoding.  No blocking,
fusion or reordering beyond what the definitions state.

Citations name the source pages by these short tags:

[BioNeMo]   "NVIDIA发布BioNeMo MoE配方：八卡B200训练Mixtral-8x7B吞吐提升至Hugging
            Face基线 2.21 倍" (scopeai.cc story on NVIDIA's "Efficient MoE
            Training for Biological Foundation Models"); sections
            "MoE训练的瓶颈与TE的对应能力" (bottlenecks), "GroupedLinear"
            (grouped GEMM), "MXFP8与融合MLP" (MXFP8 and the fused MLP).
[AutoModel] "英伟达开源MoE加速神器：一行代码，微调快3.7倍" (openai-hub.com);
            sections "MoE 微调的痛点" (sparse activation), "专家并行" (expert
            parallelism: dispatch to experts, compute, send back).

Modules:
  mx     -- E4M3 element / E8M0 block-scale encoding, rowwise and grouped
            columnwise block layouts, dequantization.
  route  -- top-k routing, split sizes, stable permutation, permute /
            unpermute, routing backward.
  mlp    -- grouped gate_up -> ScaledSwiGLU -> down, forward and backward,
            in BF16 and MXFP8, and the full layer step.
  router -- the router linear layer (logits = X W_r^T) in front of the
            routing, its backward, and the layer step with it.

Parity status of each function is stated in its docstring; the conventions the
pages leave open (gate/up half order, softmax over the selected k) are marked
"parity unpinned" where no pin beyond internal consistency exists.
"""
from . import mx, route, mlp, router  # noqa: F401
