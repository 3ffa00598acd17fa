"""GPU parity of the FP8 matrix-core path against its oracle (page [P537] §9.2: Q, K,
V in E4M3 with one power-of-two scale per 128 elements): the row quantizer bit for
bit, then tree_verify_attention_fp8 element by element."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_mma as M

pytestmark = pytest.mark.gpu


def quant_rows_case(rng, rows: int) -> np.ndarray:
    """fp32 rows spanning the awkward cases of the scale rule and the rounding."""
    x = rng.normal(0, 1, (rows, 128)).astype(np.float32)
    x *= np.exp(rng.normal(0, 4, (rows, 1))).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2] = 0.0
    x[2, 7] = -3.5
    x[3] = 448.0 * 2.0 ** np.arange(-64, 64).astype(np.float32)[:128]
    x[4] = 1e-39                          # fp32 subnormal row
    x[4, ::3] = -1e-40
    x[5] = np.float32(448.0) * np.float32(1 + 2**-23)
    vals = oracle.e4m3_table()[:0x7F]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x[6] = np.concatenate([mids, [448.0, 1.0]]).astype(np.float32)  # every tie, row max 448
    x[7] = -x[6]
    return x


@pytest.mark.parametrize("rows", [1, 13, 1000, 4097])
def test_quantize_rows_fp32_bitexact(gpu_lib, rows):
    rng = np.random.default_rng(rows)
    x = quant_rows_case(rng, max(rows, 8))[:rows] if rows < 8 else quant_rows_case(rng, rows)
    codes, exps = gpu_lib.tree_quantize_rows_e4m3(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    want_c, want_e = M.quantize_rows(x)
    np.testing.assert_array_equal(exps.cpu().numpy(), want_e)
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)


@pytest.mark.parametrize("rows", [7, 2048])
def test_quantize_rows_bf16_bitexact(gpu_lib, rows):
    rng = np.random.default_rng(100 + rows)
    x = quant_rows_case(rng, max(rows, 8))[:rows]
    xb = torch.from_numpy(x).to(torch.bfloat16)
    codes, exps = gpu_lib.tree_quantize_rows_e4m3(xb.cuda())
    torch.cuda.synchronize()
    want_c, want_e = M.quantize_rows(xb.float().numpy())
    np.testing.assert_array_equal(exps.cpu().numpy(), want_e)
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)


def test_quantize_rows_shapes(gpu_lib):
    x = torch.randn(3, 5, 128, device="cuda", dtype=torch.bfloat16)
    codes, exps = gpu_lib.tree_quantize_rows_e4m3(x)
    assert codes.shape == (3, 5, 128) and exps.shape == (3, 5)
    empty_c, empty_e = gpu_lib.tree_quantize_rows_e4m3(torch.empty(0, 128, device="cuda"))
    assert empty_c.numel() == 0 and empty_e.numel() == 0
