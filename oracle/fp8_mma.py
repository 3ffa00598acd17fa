"""FP8 matrix-core attention oracle: Q, K and V in E4M3 with power-of-two row scales
— TEST INFRASTRUCTURE ONLY (see the package docstring).

Page [P537] "端云协同推测解码中草稿模型动态生成与验证并行化…", §9.2 (FP8 mixed-precision
tree attention): Q, K and V are held in FP8 E4M3 with block scaling, one scale per
block of 128 elements, and the accumulators stay fp32; appendix B passes the block
scales beside Q, K and V and applies them when a block is loaded.

Readings taken where the page leaves the step open (each also in the design notes):
  * Every 128-element row (one head of one token, head_dim 128) is one block:
    the rows of Q, of the tree's K and V, and of the paged K/V cache.
  * Scales are powers of two stored as one E8M0 byte e (value 2^(e - 127), e in
    0..254): the microscaling scale format that gfx950's scaled FP8 matrix
    instructions consume, so a scale costs no arithmetic.
  * Quantizing a row x (fp32 values): amax = max |x|; its scale is the smallest
    power of two 2^s with amax <= 448 * 2^s (448 = largest finite E4M3), s in
    [-127, 127]; an all-zero row takes s = 0.  Codes = round-to-nearest-even of
    x * 2^-s to E4M3 (the product is exact).  K and V, the paged prefix and the
    tree's own rows alike, arrive in this format (codes and exponent bytes: the
    forward pass that writes the FP8 cache writes the tree's K/V the same way);
    Q arrives in bf16 and is quantized by this rule inside the step.
  * Attention is then the plain definition (oracle.attention) over the
    dequantized values, code value * 2^s, in fp64.

Pins (tests/test_oracle_fp8_mma.py): E4M3 rounding equals torch's float8_e4m3fn
cast, including every tie; the scale rule's closed forms and its defining
property (amax * 2^-s in (224, 448]); the round trip's error bound; exact inputs
reduce to the fp32-scale FP8 oracle and to plain attention.
"""
from __future__ import annotations

import numpy as np

from .attention import tree_attention
from .fp8 import e4m3_table

E4M3_MAX = 448.0


def _finite_positive_values() -> np.ndarray:
    """Values of codes 0x00 .. 0x7E (non-negative, finite), ascending."""
    return e4m3_table()[:0x7F]


def e4m3_round(x) -> np.ndarray:
    """Round-to-nearest-even of fp32 values to E4M3 codes (|x| <= 448 expected;
    larger magnitudes saturate to 448).  The sign bit follows the sign of x,
    negative zero included."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    vals = _finite_positive_values()
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(vals, mag, side="left")          # first value >= mag
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    # nearest; on a tie the code with an even mantissa (even code) wins
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(mag == vals[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def scale_shift(amax) -> np.ndarray:
    """s of the row scale 2^s: the smallest power of two with amax <= 448 * 2^s,
    s clamped to [-127, 127]; s = 0 for amax = 0.  From the fp32 bits: with
    amax = m * 2^E (1 <= m < 2), s = E - 8, plus 1 when m > 1.75 (448 = 1.75 * 2^8)."""
    a = np.asarray(amax, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.int64)
    expo = (bits >> 23) & 0xFF
    mant = bits & 0x7FFFFF
    # subnormal amax: value = mant * 2^-149; normalise it for the rule
    s = np.where(expo > 0, (expo - 127) - 8 + (mant > 0x600000), 0)
    sub = (expo == 0) & (mant > 0)
    if np.any(sub):
        m = mant[sub].astype(np.float64) * 2.0 ** -149
        e = np.floor(np.log2(m)).astype(np.int64)
        frac = m / 2.0 ** e
        s_sub = e - 8 + (frac > 1.75)
        s = s.copy()
        s[sub] = s_sub
    s = np.where((expo == 0) & (mant == 0), 0, s)
    return np.clip(s, -127, 127).astype(np.int64)


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """x [..., 128] (fp32 values) -> (codes [..., 128] uint8, exponent bytes [...] uint8)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = scale_shift(amax)
    scaled = (x.astype(np.float64) * np.exp2(-s.astype(np.float64))[..., None]).astype(np.float32)
    return e4m3_round(scaled), (s + 127).astype(np.uint8)


def dequantize_rows(codes, exps) -> np.ndarray:
    """codes [..., 128] uint8, exps [...] uint8 -> fp64 values code * 2^(e - 127)."""
    return e4m3_table()[np.asarray(codes, dtype=np.uint8)] * np.exp2(
        np.asarray(exps, dtype=np.float64) - 127.0)[..., None]


def round_trip(x) -> np.ndarray:
    """The values the matrix cores see for rows x: quantize, then dequantize."""
    return dequantize_rows(*quantize_rows(x))


def tree_attention_fp8mma(q, k8, v8, k_exp, v_exp, block_table, prefix_len, kt8, vt8, kt_exp,
                          vt_exp, cu_nodes, parent, hq: int, hkv: int, scale: float, nodes=None):
    """Tree attention with Q, K and V in E4M3 and E8M0 row scales: q [total, hq, 128]
    are the fp32 values of the bf16 queries, quantized per row here; k8 / v8
    [num_blocks, hkv, 64, 128] with k_exp / v_exp [num_blocks, hkv, 64] are the paged
    cache, kt8 / vt8 [total, hkv, 128] with kt_exp / vt_exp [total, hkv] the tree's
    K/V, all as codes and exponent bytes."""
    return tree_attention(round_trip(q), dequantize_rows(k8, k_exp), dequantize_rows(v8, v_exp),
                          block_table, prefix_len, dequantize_rows(kt8, kt_exp),
                          dequantize_rows(vt8, vt_exp), cu_nodes, parent, hq, hkv, scale,
                          nodes=nodes)
