"""CPU oracle for the tree-verification step — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct fp64 / integer implementations of what the
verify step computes.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the library itself
never routes through it, and this package shares no code with the HIP path.

Sources (cited in each function by page and section):
  [P500] "端侧多模态大模型推测解码草稿模型动态剪枝：详解基于重要性采样的树形验证并行加速策略"
         https://www.ufo.work/2026/500.html
  [P525] "端侧大模型推测解码草稿模型动态剪枝策略：详解基于重要性采样的树形验证并行加速机制"
         https://www.ufo.work/2026/525.html
  [P537] "端云协同推测解码中草稿模型动态生成与验证并行化：探究树形注意力机制与显存碎片整理联合加速"
         https://www.ufo.work/2026/537.html
  [ViSpec] "视觉语言模型加速：ViSpec框架与推测解码优化"
         https://intelliparadigm.com/article/weixin_42533910/2016197

Parity status of each function is pinned by tests under tests/ (see
test_oracle_*.py); every function here has at least one independent pin.
"""
from .tree import (ERR_BAD_PARENT, ERR_TOO_MANY_NODES, ERR_TOKEN, ERR_BLOCK, ERR_ZERO_MASS,
                   ERR_PATH, ERR_UNIFORM, ancestors_or_self, depths, anc_bitsets, build_index)
from .attention import tree_attention
from .acceptance import accept, accept_sequence, residual_token
from .commit import commit_kv
from .probs import softmax_rows, softmax_rows_kept
from .fp8 import e4m3_table, dequantize, tree_attention_fp8
from .draft_tree import ERR_DRAFT, build_tree, build_trees
from .philox import philox4x64, uniform24, node_uniforms
from .fp8_mma import e4m3_round, scale_shift, quantize_rows, dequantize_rows, tree_attention_fp8mma

__all__ = [
    "ERR_BAD_PARENT", "ERR_TOO_MANY_NODES", "ERR_TOKEN", "ERR_BLOCK", "ERR_ZERO_MASS",
    "ERR_PATH", "ERR_UNIFORM", "ancestors_or_self", "depths", "anc_bitsets", "build_index",
    "tree_attention", "accept", "accept_sequence", "residual_token", "commit_kv",
    "softmax_rows", "softmax_rows_kept", "e4m3_table", "dequantize", "tree_attention_fp8", "ERR_DRAFT", "build_tree",
    "build_trees", "philox4x64", "uniform24", "node_uniforms", "e4m3_round", "scale_shift",
    "quantize_rows", "dequantize_rows", "tree_attention_fp8mma",
]
