"""CPU oracle for the one-GPU Mixture-of-Experts layer.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import or call anything in this package.  The HIP
library never calls it, and it imports nothing from the HIP library: the two share no code.

Everything here is plain float64 numpy, written from the pages' description of the layer:

* the MoE forward pseudo-code on the cloud.baidu.com page "MoE架构的物理瓶颈与扩展限制解析"
  (section "工作原理": gate network -> top-k -> dispatch -> local expert compute -> combine);
* the five-step fused-kernel list on the apxml.com page "硬件加速的考量" (section
  "自定义核与核融合": gate scores, top-k, gather, expert matmuls, gate-weighted combine);
* the SonicMoE summary page (hebangwen.github.io, "SonicMoE: 加速 MoE 模型的 IO 与 Tile 感知优化"):
  optimization 1 (recompute instead of caching, same mathematics), optimization 3 (token rounding),
  "反向传播优化" (which operands each backward GEMM gathers) and the kernel-comparison table
  (SwiGLU fusion, dS computation, no separate scatter kernel).

``oracle/fp8.py`` adds the FP8 (OCP E4M3) row quantisation and the quantised expert FFN, and
``oracle/mx.py`` the block-scaled variant (E4M3 or E5M2 elements, one power-of-two scale per 32
elements along K), both from the apxml.com page's section "利用稀疏性和量化" (quantisation of
weights and activations).

Where the pages leave a step open, the reading taken is stated at the function that takes it.
Every function's result is pinned by tests under ``tests/`` (brute force, closed forms,
invariants, finite differences, autograd); see ``tests/test_oracle_*.py``.
"""

from .moe import (  # noqa: F401
    ROUND_NONE, ROUND_NEAREST, ROUND_UP, ROUND_DOWN,
    router_logits, topk_select, plain_topk_weights, token_rounding, gate_weights,
    build_plan, permute, unpermute, combine,
    swiglu_expert_forward, layer_forward, token_forward, layer_backward, router_backward,
)
