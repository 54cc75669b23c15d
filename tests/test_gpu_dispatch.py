"""GPU parity across the schedule boundaries of every product entry point.

Each entry point picks its kernel from M and from how many column tiles the
product has against the CU count (decode kernels up to 32 or 64 rows, the
panel schedule for one row of tiles short of the CUs, 128-row tiles, 256-row
panels, persistent 256-row tiles from 385 or 513 rows).  This sweep runs M on
both sides of every such boundary, at a narrow width, a width of about one
32-column panel per CU, and a width wide enough for the 64-column and 256-row
choices; K = 72 (one full 64-deep block and a ragged one; 80 for FP8, whose
K is a multiple of 16 and whose blocks are 128 deep).  Every element is
compared with the oracle: the bf16 product (packed, interleaved and row-major
entry points) and the FP8 product with the tolerance of the parity tests, the
packed GEMM within one bf16 rounding flip."""
import numpy as np
import pytest
import torch

import oracle
import swiglu_gated_mlp_amd as sw
from swiglu_gated_mlp_amd import inputs

from _util import check_close, f32, gpu_bits, say

pytestmark = pytest.mark.gpu

K = 72
K8 = 80
ROWS = [1, 8, 9, 16, 17, 32, 33, 64, 65, 128, 129, 192, 255, 256, 257, 384, 385, 448, 512, 513, 640]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sw.lib()
    oracle.set_threads(16)
    return torch.device("cuda:0")


def _width(name: str) -> int:
    cus = sw.swiglu_device_cu_count()
    return {"narrow": 520,                                  # 5 packed tiles, 17 panels
            "per-cu": 32 * cus - 24,                        # about one 32-column panel per CU
            "wide": 64 * ((3 * cus + 1) // 2) + 40}[name]   # >= 1.5 64-column workgroups per CU


def _gemm_close(got_bits, ref_bits, what):
    got = f32(got_bits).astype(np.float64)
    ref = f32(ref_bits).astype(np.float64)
    bad = np.argwhere(np.abs(got - ref) > 2.0 ** -7 * np.abs(ref) + 1e-3)
    assert bad.size == 0, "%s: %d elements beyond 1 ulp, e.g. %s" % (what, len(bad), bad[0].tolist())


@pytest.mark.parametrize("width", ["narrow", "per-cu", "wide"])
@pytest.mark.parametrize("M", ROWS)
def test_bf16_entry_points(dev, M, width):
    N = _width(width)
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=7 * M + N)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    out = {}
    say("[dispatch bf16] M=%d K=%d N=%d packed" % (M, K, N))
    out["packed"] = sw.swiglu_fused_packed(Ad, sw.swiglu_pack_weights(W1d, W2d), N)
    say("[dispatch bf16] M=%d K=%d N=%d interleaved" % (M, K, N))
    out["interleaved"] = sw.swiglu_fused_packed_interleaved(Ad, sw.swiglu_pack_weights_interleaved(W1d, W2d), N)
    say("[dispatch bf16] M=%d K=%d N=%d row-major" % (M, K, N))
    out["row-major"] = sw.swiglu_fused(Ad, W1d, W2d)
    torch.cuda.synchronize()
    ref = oracle.swiglu(A, W1, W2)
    for name, y in out.items():
        check_close(gpu_bits(y), ref, "%s %s" % (name, (M, K, N)))


@pytest.mark.parametrize("width", ["narrow", "per-cu", "wide"])
@pytest.mark.parametrize("M", ROWS)
def test_fp8_entry_point(dev, M, width):
    N = _width(width)
    A8, W18, W28, sg, su = inputs.fp8_case(M, K8, N, seed=5 * M + N)
    say("[dispatch fp8] M=%d K=%d N=%d" % (M, K8, N))
    Wp = sw.swiglu_pack_weights_fp8(W18.to(dev), W28.to(dev))
    Y = sw.swiglu_fused_packed_fp8(A8.to(dev), Wp, N, sg, su)
    torch.cuda.synchronize()
    ref = oracle.swiglu_fp8(A8.numpy(), W18.numpy(), W28.numpy(), sg, su)
    check_close(gpu_bits(Y), ref, "fp8 %s" % ((M, K8, N),))


@pytest.mark.parametrize("width", ["narrow", "per-cu", "wide"])
@pytest.mark.parametrize("M", ROWS)
def test_gemm_entry_points(dev, M, width):
    N = _width(width)
    A, W, _ = inputs.gaussian_case(M, K, N, seed=11 * M + N)
    Ad, Wd = A.to(dev), W.to(dev)
    say("[dispatch gemm] M=%d K=%d N=%d packed" % (M, K, N))
    Cp = sw.swiglu_gemm_packed(Ad, sw.swiglu_gemm_pack_weight(Wd), N)
    say("[dispatch gemm] M=%d K=%d N=%d row-major" % (M, K, N))
    Cr = sw.swiglu_gemm_bf16(Ad, Wd)
    torch.cuda.synchronize()
    ref = oracle.gemm_bf16(A, W)
    _gemm_close(gpu_bits(Cp), ref, "gemm packed %s" % ((M, K, N),))
    _gemm_close(gpu_bits(Cr), ref, "gemm row-major %s" % ((M, K, N),))
