"""swiglu_fused_packed_noalloc: the split-K partial sums in the library's own
device scratch array instead of a caller's workspace.  Checked against
swiglu_fused_packed (same schedule, so bit for bit) and against the oracle,
on calls in a row on one device, the later ones smaller, so the array holds
the earlier call's partial sums when the next one starts."""
import numpy as np
import pytest
import torch

import oracle
import swiglu_gated_mlp_amd as sw
from swiglu_gated_mlp_amd import inputs

from _util import check_close, gpu_bits, say

pytestmark = pytest.mark.gpu

SPLIT, AUTO, DP = sw.VARIANT_SPLIT_K, sw.VARIANT_AUTO, sw.VARIANT_DATA_PARALLEL


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sw.lib()
    oracle.set_threads(16)
    return torch.device("cuda:0")


def _allocations():
    return torch.cuda.memory_stats().get("allocation.all.allocated", 0)


@pytest.mark.parametrize("variant", [SPLIT, AUTO])
def test_noalloc_matches_workspace_entry_point(dev, variant):
    # (M, K, N): the first call's split-K partial sums fill about half of the
    # scratch array, the next calls are smaller (ragged K and N on the last)
    shapes = [(64, 4096, 1024), (16, 1024, 512), (40, 200, 264)]
    for i, (M, K, N) in enumerate(shapes):
        need = sw.swiglu_workspace_bytes(M, K, N, variant)
        if variant == SPLIT:
            assert 0 < need <= sw.NOALLOC_SCRATCH_BYTES, (M, K, N, need)
        A, W1, W2 = inputs.gaussian_case(M, K, N, seed=900 + i)
        Ad, Wp = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        say("[noalloc] call %d M=%d K=%d N=%d variant=%d scratch bytes=%d" % (i, M, K, N, variant, need))
        before = _allocations()
        sw.swiglu_fused_packed_noalloc(Ad, Wp, Y, variant=variant)
        assert _allocations() == before, "the no-allocation call allocated through torch"
        Yw = sw.swiglu_fused_packed(Ad, Wp, N, variant=variant)
        torch.cuda.synchronize()
        got, want = gpu_bits(Y), gpu_bits(Yw)
        assert np.array_equal(got, want), "call %d: noalloc != swiglu_fused_packed bitwise" % i
        check_close(got, oracle.swiglu(A, W1, W2), "noalloc call %d %s" % (i, (M, K, N)))


def test_noalloc_rejects_oversized_partials(dev):
    # split-K at the 7B width and 128 rows: two or more splits of 128 x 2N
    # fp32 partial sums, beyond the scratch array
    M, K, N = 128, 3584, 18944
    need = sw.swiglu_workspace_bytes(M, K, N, SPLIT)
    assert need > sw.NOALLOC_SCRATCH_BYTES
    A = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    Wp = torch.zeros(sw.swiglu_packed_bytes(K, N) // 2, dtype=torch.bfloat16, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    with pytest.raises(sw.SwigluError) as ei:
        sw.swiglu_fused_packed_noalloc(A, Wp, Y, variant=SPLIT)
    assert ei.value.status == 6
    # the data-parallel schedule of the same shape needs no scratch
    sw.swiglu_fused_packed_noalloc(A, Wp, Y, variant=DP)
    torch.cuda.synchronize()
    assert torch.all(Y.float() == 0)
