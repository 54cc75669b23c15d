"""GPU parity on seeded random shapes through every product entry point.

The hand-picked shapes elsewhere sit on the schedules' boundaries; these draw
M, K and N at random (K and N multiples of 8, K of 16 for FP8, some products
wide enough for the many-column schedules) so that combinations nobody chose
are exercised too.  Every element is compared with the oracle: the bf16
product (packed AUTO, forced split-K, interleaved and row-major entry points)
and the FP8 product within the parity tolerance, the packed and row-major
GEMMs within one bf16 rounding flip."""
import numpy as np
import pytest
import torch

import oracle
import swiglu_gated_mlp_amd as sw
from swiglu_gated_mlp_amd import inputs

from _util import check_close, f32, gpu_bits, say

pytestmark = pytest.mark.gpu


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = max(1, int(np.exp(rng.uniform(0.0, np.log(700.0)))))   # log-uniform: decode sizes too
        if i % 4 == 3:      # wide and shallow: the many-column schedules
            K = 16 * int(rng.integers(1, 12))
            N = 8 * int(rng.integers(1500, 4200))
        else:
            K = 16 * int(rng.integers(1, 40))
            N = 8 * int(rng.integers(1, 400))
        out.append((M, K, N))
    return out


SHAPES = _shapes(64, 2024)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sw.lib()
    oracle.set_threads(16)
    return torch.device("cuda:0")


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_random_shape(dev, M, K, N):
    seed = M * 7 + K * 3 + N
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=seed)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    say("[random] M=%d K=%d N=%d" % (M, K, N))
    Wp = sw.swiglu_pack_weights(W1d, W2d)
    out = {
        "auto": sw.swiglu_fused_packed(Ad, Wp, N),
        "split": sw.swiglu_fused_packed(Ad, Wp, N, variant=sw.VARIANT_SPLIT_K),
        "interleaved": sw.swiglu_fused_packed_interleaved(Ad, sw.swiglu_pack_weights_interleaved(W1d, W2d), N),
        "row-major": sw.swiglu_fused(Ad, W1d, W2d),
    }
    Cp = sw.swiglu_gemm_packed(Ad, sw.swiglu_gemm_pack_weight(W1d), N)
    Cr = sw.swiglu_gemm_bf16(Ad, W1d)
    A8, W18, W28, sg, su = inputs.fp8_case(M, K, N, seed=seed)
    Y8 = sw.swiglu_fused_packed_fp8(A8.to(dev), sw.swiglu_pack_weights_fp8(W18.to(dev), W28.to(dev)), N, sg, su)
    torch.cuda.synchronize()
    ref = oracle.swiglu(A, W1, W2)
    for name, y in out.items():
        check_close(gpu_bits(y), ref, "%s %s" % (name, (M, K, N)))
    check_close(gpu_bits(Y8), oracle.swiglu_fp8(A8.numpy(), W18.numpy(), W28.numpy(), sg, su),
                "fp8 %s" % ((M, K, N),))
    g = oracle.gemm_bf16(A, W1)
    for name, c in (("gemm packed", Cp), ("gemm row-major", Cr)):
        got = f32(gpu_bits(c)).astype(np.float64)
        want = f32(g).astype(np.float64)
        bad = np.argwhere(np.abs(got - want) > 2.0 ** -7 * np.abs(want) + 1e-3)
        assert bad.size == 0, "%s %s: %d elements beyond 1 ulp" % (name, (M, K, N), len(bad))
