"""HIP graph capture of the fused entry points: every schedule enqueues only
kernel launches (no allocation, no memset, no synchronisation), so a captured
call replays correctly.  Each graph is replayed several times with the
program's own eager work and synchronisations in between, and every replay is
checked bitwise against an eager call on the same inputs, also after the
inputs change in place."""
import numpy as np
import pytest
import torch

import swiglu_gated_mlp_amd as sw
from swiglu_gated_mlp_amd import inputs

from _util import gpu_bits, say

pytestmark = pytest.mark.gpu

DP, SPLIT, AUTO, DECODE = (sw.VARIANT_DATA_PARALLEL, sw.VARIANT_SPLIT_K, sw.VARIANT_AUTO,
                           sw.VARIANT_DECODE)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sw.lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("M,K,N,variant", [
    (16, 896, 4864, AUTO),        # decode kernel
    (64, 896, 4864, AUTO),        # decode kernel, four row tiles per workgroup
    (128, 512, 4096, AUTO),       # panel schedule
    (300, 136, 264, DP),          # 128-row tiles, ragged K
    (4096, 896, 4864, AUTO),      # persistent 256-row grid + 128-row tail (one launch)
    (128, 2048, 1024, SPLIT),     # split-K: partials to the workspace, then the reduction
])
def test_graph_replay_matches_eager(dev, M, K, N, variant):
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=M + K + N + variant)
    A2, _, _ = inputs.gaussian_case(M, K, N, seed=M + K + N + 100)
    Ad, Wp = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    ws = sw.Workspace(dev)
    ws.get(sw.swiglu_workspace_bytes(M, K, N, variant))
    Yg = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    say("[graph] M=%d K=%d N=%d variant=%d" % (M, K, N, variant))
    # warm-up call on a side stream, then the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sw.swiglu_fused_packed(Ad, Wp, N, Y=Yg, workspace=ws, variant=variant)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.swiglu_fused_packed(Ad, Wp, N, Y=Yg, workspace=ws, variant=variant)
    torch.cuda.synchronize()
    ws_eager = sw.Workspace(dev)
    for rep, src in enumerate((A, A, A2, A2)):
        Ad.copy_(src.to(dev))                 # the graph reads A where it was captured
        Yg.fill_(0)
        g.replay()
        # the program's own eager work between replays
        Ye = sw.swiglu_fused_packed(Ad, Wp, N, workspace=ws_eager, variant=variant)
        scratch = torch.randn(1 << 16, device=dev).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert np.array_equal(gpu_bits(Yg), gpu_bits(Ye)), "replay %d differs from eager" % rep


@pytest.mark.parametrize("M,K,N", [
    (1, 3584, 1032),      # decode kernel on weight halves
    (128, 3584, 18944),   # panel schedule on half-panels
    (128, 4864, 896),     # split-K: partials to the workspace, then the GEMM's reduction
])
def test_gemm_graph_replay_matches_eager(dev, M, K, N):
    """The single-weight GEMM (the unfused pipeline's and the MLP down
    projection's) under capture, the same way."""
    A, W, _ = inputs.gaussian_case(M, K, N, seed=13 * M + K + N)
    A2, _, _ = inputs.gaussian_case(M, K, N, seed=13 * M + K + N + 100)
    Ad, Wg = A.to(dev), sw.swiglu_gemm_pack_weight(W.to(dev))
    ws = sw.Workspace(dev)
    ws.get(sw.swiglu_gemm_workspace_bytes(M, K, N))
    Cg = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    say("[graph gemm] M=%d K=%d N=%d workspace=%d" % (M, K, N, sw.swiglu_gemm_workspace_bytes(M, K, N)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sw.swiglu_gemm_packed(Ad, Wg, N, C=Cg, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.swiglu_gemm_packed(Ad, Wg, N, C=Cg, workspace=ws)
    torch.cuda.synchronize()
    ws_eager = sw.Workspace(dev)
    for rep, src in enumerate((A, A, A2, A2)):
        Ad.copy_(src.to(dev))
        Cg.fill_(0)
        g.replay()
        Ce = sw.swiglu_gemm_packed(Ad, Wg, N, workspace=ws_eager)
        scratch = torch.randn(1 << 16, device=dev).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert np.array_equal(gpu_bits(Cg), gpu_bits(Ce)), "replay %d differs from eager" % rep
