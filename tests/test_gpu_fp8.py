"""GPU parity of the FP8 (E4M3, per-tensor scales) path against the oracle's
swiglu_fp8, through the C ABI: the packed layout byte by byte, then the
product on every streaming schedule (panel, 128-row tiles, persistent
256-row tiles, the mixed 256/128-row launch) with ragged K and N, and
sampled rows at the workload shapes.  Tolerance as everywhere:
|y - ref| <= 1e-3 + 8e-3 |ref| (the sums differ only in fp32 order; every
E4M3 product is exact in fp32)."""
import numpy as np
import pytest
import torch

import oracle
import swiglu_gated_mlp_amd as sw
from swiglu_gated_mlp_amd import inputs

from _util import cached_oracle, check_close, check_close_all, gpu_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sw.lib()
    oracle.set_threads(16)
    return torch.device("cuda:0")


def test_fp8_pack_layout(dev):
    for K, N in [(128, 128), (144, 136), (896, 520)]:
        g = torch.Generator().manual_seed(K + N)
        W1 = torch.randint(0, 256, (K, N), generator=g, dtype=torch.uint8)
        W2 = torch.randint(0, 256, (K, N), generator=g, dtype=torch.uint8)
        P = sw.swiglu_pack_weights_fp8(W1.to(dev), W2.to(dev)).cpu().numpy()
        KB = (K + 127) // 128
        assert P.size == ((N + 127) // 128) * KB * 32768

        def pos(jt, kb, prow, k):
            # [rb][64-k step ks][half of the lane's 32 bytes][lane = 32 h + r][16 bytes]
            rb, r, ks, h, j = prow // 32, prow % 32, k // 64, (k % 64) // 32, k % 32
            return (jt * KB + kb) * 32768 + (((rb * 2 + ks) * 2 + j // 16) * 64 + h * 32 + r) * 16 + j % 16

        w1, w2 = W1.numpy(), W2.numpy()
        rng = np.random.default_rng(K)
        for _ in range(400):
            n, k = int(rng.integers(0, N)), int(rng.integers(0, K))
            jt, c = n // 128, n % 128
            assert P[pos(jt, k // 128, c, k % 128)] == w1[k, n]
            assert P[pos(jt, k // 128, 128 + c, k % 128)] == w2[k, n]
        JT = (N + 127) // 128
        for c in range(N % 128 or 128, 128, 5):
            assert P[pos(JT - 1, 0, c, 3)] == 0 and P[pos(JT - 1, 0, 128 + c, 70)] == 0
        if K % 128:
            for n in range(0, N, 13):
                for k in range(K % 128, 128, 11):
                    assert P[pos(n // 128, KB - 1, n % 128, k)] == 0


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 128),         # FP8 decode kernel: one row, half a block
    (16, 208, 2056),      # FP8 decode, activations via LDS: ragged K, a partial last column group
    (32, 1024, 8192),     # FP8 decode, activations via LDS, 32 rows
    (7, 3584, 18944),     # FP8 decode at the 7B width, one column group per workgroup
    (24, 1024, 29568),    # FP8 decode at the 72B width: four column groups per workgroup
    (40, 208, 520),       # panel schedule, ragged K, partial last column tile
    (128, 512, 4096),     # panel schedule, 2-3 panels per workgroup
    (200, 256, 16392),    # two rows of 128-row tiles, wide: one row of 256-row tiles on the panel schedule
    (300, 144, 264),      # 128-row tiles, ragged K
    (2100, 128, 256),     # persistent 256-row tiles, M tail
    (4000, 256, 2696),    # mixed 256/128-row launch, partial last column tile
])
def test_fp8_parity(dev, M, K, N):
    A8, W18, W28, sg, su = inputs.fp8_case(M, K, N, seed=M + K + N)
    say("[fp8] M=%d K=%d N=%d" % (M, K, N))
    Wp = sw.swiglu_pack_weights_fp8(W18.to(dev), W28.to(dev))
    Y = gpu_bits(sw.swiglu_fused_packed_fp8(A8.to(dev), Wp, N, sg, su))
    ref = oracle.swiglu_fp8(A8.numpy(), W18.numpy(), W28.numpy(), sg, su)
    check_close(Y, ref, "fp8 %s" % ((M, K, N),))


@pytest.mark.parametrize("name,M", [(w.name, m) for w in inputs.WORKLOADS for m in w.ms],
                         ids=["%s-M%d" % (w.name, m) for w in inputs.WORKLOADS for m in w.ms])
def test_fp8_workload_shapes(dev, name, M):
    """The workload's own tensors quantised per tensor, at every workload
    point (decode kernel up to 32 rows, the tiny point's panel schedule, the
    mixed prefill launch); every element against the oracle."""
    w = inputs.BY_NAME[name]
    A, W1, W2 = inputs.workload_tensors(w, M)
    A8, sa = inputs.quantize_e4m3(A)
    W18, s1 = inputs.quantize_e4m3(W1)
    W28, s2 = inputs.quantize_e4m3(W2)
    sg = float(np.float32(sa) * np.float32(s1))
    su = float(np.float32(sa) * np.float32(s2))
    say("[fp8-workload] %s M=%d" % (name, M))
    Wp = sw.swiglu_pack_weights_fp8(W18.to(dev), W28.to(dev))
    Y = gpu_bits(sw.swiglu_fused_packed_fp8(A8.to(dev), Wp, w.N, sg, su))
    ref = cached_oracle("fp8-%s-M%d" % (name, M),
                        lambda: oracle.swiglu_fp8(A8.numpy(), W18.numpy(), W28.numpy(), sg, su))
    idx = check_close_all(Y, ref, "fp8 %s" % name)
    say("  all %d elements within tolerance; bitwise mismatch %.5f%%" % (ref.size, 100 * idx.size / ref.size))
