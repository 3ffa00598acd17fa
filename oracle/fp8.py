"""FP8 (E4M3) key/value cache oracle: decoding, dequantization, attention.

The pages move attention's Q, K and V to FP8 E4M3 with block scaling (one
scale shared by each block of 128 elements) while the accumulators stay fp32
(page [P537] "端云协同推测解码中草稿模型动态生成与验证并行化…", §9.2, FP8 mixed-
precision tree attention; appendix B, the block scales passed beside Q, K and V
and applied when a block is loaded).

Readings taken where the pages leave the step open:
  * The FP8 format is OCP E4M3 ("fn": 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals, no infinities, S.1111.111 is NaN, largest finite 448).
  * Only the paged prefix cache is FP8: it is what the verify step streams from
    HBM, so it is what halving the element size pays for.  Q and the tree's own
    K/V are produced fresh by this step's forward pass and stay bf16.
  * A block of 128 elements is one (cache block, KV head, position) row of
    head_dim = 128: scale[num_blocks, hkv, 64], fp32, value = e4m3 * scale.
  * Dequantization is exact (fp64 here); attention is then the plain definition
    of oracle.attention on the dequantized cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .attention import tree_attention


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 byte, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:                       # subnormal: (m / 8) * 2^(1 - 7)
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_table() -> np.ndarray:
    """The 256 byte values in fp64 (index = byte)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequantize(cache8: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """cache8 [num_blocks, hkv, 64, d] uint8, scale [num_blocks, hkv, 64] -> fp64 values."""
    return e4m3_table()[np.asarray(cache8, dtype=np.uint8)] * np.asarray(scale, dtype=np.float64)[..., None]


def tree_attention_fp8(q, k8, v8, k_scale, v_scale, block_table, prefix_len, k_tree, v_tree,
                       cu_nodes, parent, hq: int, hkv: int, scale: float, nodes=None):
    """Tree attention over an FP8 prefix cache: dequantize, then the plain
    definition.  q, k_tree, v_tree are fp64 arrays of the stored values."""
    return tree_attention(q, dequantize(k8, k_scale), dequantize(v8, v_scale), block_table,
                          prefix_len, k_tree, v_tree, cu_nodes, parent, hq, hkv, scale, nodes=nodes)
