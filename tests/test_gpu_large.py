"""Products whose activations pass 2 GiB: the library runs them as row chunks
(the streaming kernel addresses an activation tile with 32-bit offsets).
Rows on both sides of every chunk boundary and the last row are checked
against the oracle, for the bf16 (both orders), interleaved-layout and FP8
entry points.
The activations are drawn on the GPU (seeded); only the sampled rows go to
the oracle."""
import numpy as np
import pytest
import torch

import oracle
import swiglu_gated_mlp_amd as sw
from swiglu_gated_mlp_amd import inputs

from _util import check_close, gpu_bits, say

pytestmark = pytest.mark.gpu

K, N = 16384, 256


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sw.lib()
    return torch.device("cuda:0")


def _rows(M, limit):
    """Rows on both sides of the library's chunk boundaries (equal chunks,
    multiples of 256 rows, at most `limit` rows) and the last row."""
    n = -(-M // limit)
    chunk = min(limit, -(-(-(-M // n)) // 256) * 256)
    r = {0, M - 1}
    for b in range(chunk, M, chunk):
        r |= {b - 1, b}
    return sorted(r)


def _activation(dev, M, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    return torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16)


def test_bf16_over_2gib(dev):
    M = 65536 + 464                     # 2^31 / (K * 2) = 65536 rows per chunk
    Ad = _activation(dev, M, 11)
    _, W1, W2 = inputs.gaussian_case(1, K, N, seed=12)
    W1d, W2d = W1.to(dev), W2.to(dev)
    say("[large] bf16 M=%d K=%d N=%d (%.2f GiB of activations)" % (M, K, N, M * K * 2 / 2 ** 30))
    Wp = sw.swiglu_pack_weights(W1d, W2d)
    Y = gpu_bits(sw.swiglu_fused_packed(Ad, Wp, N))
    Ys = gpu_bits(sw.swiglu_fused_packed(Ad, Wp, N, variant=sw.VARIANT_SEQUENTIAL))
    Yi = gpu_bits(sw.swiglu_fused_packed_interleaved(Ad, sw.swiglu_pack_weights_interleaved(W1d, W2d), N))
    rows = _rows(M, 65536)
    A_rows = inputs.as_bits(Ad[rows].cpu())
    ref = oracle.swiglu(A_rows, W1, W2)
    check_close(Y[rows], ref, "bf16 chunked rows %s" % rows)
    assert np.array_equal(Yi, Y), "interleaved layout != per-tile layout bitwise"
    assert np.array_equal(Ys, Y), "sequential order != data-parallel bitwise"


def test_fp8_over_2gib(dev):
    M = 131072 + 200                    # 2^31 / K = 131072 rows per chunk
    A8, sa = inputs.quantize_e4m3(_activation(dev, M, 21))
    _, W1, W2 = inputs.gaussian_case(1, K, N, seed=22)
    W18, s1 = inputs.quantize_e4m3(W1)
    W28, s2 = inputs.quantize_e4m3(W2)
    sg = float(np.float32(sa) * np.float32(s1))
    su = float(np.float32(sa) * np.float32(s2))
    say("[large] fp8 M=%d K=%d N=%d (%.2f GiB of activations)" % (M, K, N, M * K / 2 ** 30))
    Wp = sw.swiglu_pack_weights_fp8(W18.to(dev), W28.to(dev))
    Y = gpu_bits(sw.swiglu_fused_packed_fp8(A8, Wp, N, sg, su))
    rows = _rows(M, 131072)
    ref = oracle.swiglu_fp8(A8[rows].cpu().numpy(), W18.numpy(), W28.numpy(), sg, su)
    check_close(Y[rows], ref, "fp8 chunked rows %s" % rows)
