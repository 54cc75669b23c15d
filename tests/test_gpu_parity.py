"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Acceptance rule (tolerance written here, used everywhere): for every compared
element |y - ref| <= 1e-3 + 8e-3 |ref|, y = GPU bf16, ref = oracle bf16.
Bitwise equality is required where the arithmetic fixes the result exactly
(integer regime, invariants, determinism, packed == unpacked).
"""
import numpy as np
import pytest
import torch

import oracle
import swiglu_gated_mlp_amd as sw
from swiglu_gated_mlp_amd import inputs

from _util import (PageMetric, cached_oracle, check_close, check_close_all, diff_positions, f32, gpu_bits,
                   mismatch_rates, oracle_rows, sample_rows, say)

pytestmark = pytest.mark.gpu

DP, SPLIT, AUTO, DECODE, SEQ = (sw.VARIANT_DATA_PARALLEL, sw.VARIANT_SPLIT_K, sw.VARIANT_AUTO,
                                sw.VARIANT_DECODE, sw.VARIANT_SEQUENTIAL)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sw.lib()
    oracle.set_threads(16)
    return torch.device("cuda:0")


def run_all_variants(dev, A, W1, W2, label):
    """Y from swiglu_fused and swiglu_fused_packed under every schedule."""
    M, K = A.shape
    N = W1.shape[1]
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    Wp = sw.swiglu_pack_weights(W1d, W2d)
    out = {}
    say("[%s] M=%d K=%d N=%d fused" % (label, M, K, N))
    out["fused"] = sw.swiglu_fused(Ad, W1d, W2d)
    variants = [("dp", DP), ("split", SPLIT), ("auto", AUTO), ("seq", SEQ)]
    if M <= 64:
        variants.append(("decode", DECODE))
    for name, v in variants:
        say("[%s] M=%d K=%d N=%d packed/%s" % (label, M, K, N, name))
        out[name] = sw.swiglu_fused_packed(Ad, Wp, N, variant=v)
    torch.cuda.synchronize()
    bits = {k: gpu_bits(v) for k, v in out.items()}
    # the sequential order sums the same MFMAs in the same order as the dual
    # loop of the data-parallel schedule
    assert np.array_equal(bits["seq"], bits["dp"]), "sequential != data-parallel bitwise"
    return bits


SMALL_SHAPES = [
    (1, 64, 128), (3, 72, 136), (17, 200, 256), (32, 128, 128), (33, 64, 264), (63, 128, 384),
    (65, 896, 512), (128, 512, 256), (130, 256, 264), (255, 192, 128), (257, 512, 640),
    (300, 136, 520), (2049, 128, 256), (2100, 64, 136),
    (2304, 128, 3840),   # 270 tiles of 256x128: the last column tiles run as 128x128 tiles
    # streaming prefill kernel: ragged K (zero-chunk activation loads) with each
    # ring phase, 128- and 256-row tiles, M tails
    (200, 328, 384), (2600, 520, 256), (3000, 456, 640),
    # 352 tiles of 256x128: the last 6 column tiles run as 128-row tiles in the
    # same launch; partial last column tile, M tail, ragged K
    (4000, 200, 2696),
    # 128-row tiles, one workgroup per tile, more tiles than CUs; M and N
    # tails, ragged K (the persistent multi-tile walk of the 256-row tiles is
    # test_persistent_multi_tile_walk)
    (1500, 328, 3000), (2048, 896, 4864),
    # the smallest legal K and N (one 16-byte chunk of k; one 8-column piece of
    # a 128-column tile) on the decode, 128-row and 256-row schedules
    (3, 8, 8), (70, 8, 24), (300, 24, 8), (2100, 8, 8),
    # 256-row tiles below 2048 rows: from 385 rows with a last row tile at
    # least three quarters full and a 256-row grid that fills the CUs (with the
    # 128-row tail), and above 512 rows; 416 rows stays on 128-row tiles
    (450, 136, 18000), (512, 64, 16384), (600, 136, 2000), (416, 200, 18944),
]


@pytest.mark.parametrize("M,K,N", SMALL_SHAPES)
def test_small_shapes_every_variant(dev, M, K, N):
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=M * 7 + K + N)
    outs = run_all_variants(dev, A, W1, W2, "small")
    ref = oracle.swiglu(A, W1, W2)
    for name, y in outs.items():
        check_close(y, ref, "%s M=%d K=%d N=%d" % (name, M, K, N))
    # same MFMA chain per element: unpacked and packed data-parallel agree bitwise
    assert np.array_equal(outs["fused"], outs["dp"]), "fused != fused_packed(dp) bitwise"


def test_pack_roundtrip_and_layout(dev):
    for K, N in [(64, 128), (72, 136), (896, 4864), (200, 520)]:
        _, W1, W2 = inputs.gaussian_case(1, K, N, seed=K + N)
        W1d, W2d = W1.to(dev), W2.to(dev)
        Wp = sw.swiglu_pack_weights(W1d, W2d)
        V1, V2 = sw.swiglu_unpack_weights(Wp, K, N)
        torch.cuda.synchronize()
        assert torch.equal(V1.view(torch.int16), W1d.view(torch.int16))
        assert torch.equal(V2.view(torch.int16), W2d.view(torch.int16))
        # layout as documented in swiglu.h: tile jt, block kb, 16-row group g,
        # half h, lane l, element e
        P = inputs.as_bits(Wp.cpu())
        KB = (K + 63) // 64
        w1, w2 = inputs.as_bits(W1), inputs.as_bits(W2)

        def pos(jt, kb, g, h, l, e):
            return ((((jt * KB + kb) * 16 + g) * 2 + h) * 64 + l) * 8 + e

        rng = np.random.default_rng(K)
        for _ in range(300):
            n = int(rng.integers(0, N))
            k = int(rng.integers(0, K))
            jt, r, kb, kk = n // 128, n % 128, k // 64, k % 64
            g, h, l, e = r // 16, kk // 32, ((kk % 32) // 8) * 16 + r % 16, kk % 8
            assert P[pos(jt, kb, g, h, l, e)] == w1[k, n]
            assert P[pos(jt, kb, g + 8, h, l, e)] == w2[k, n]
        # padding is zero: columns past N in the last tile, k past K in the last block
        if N % 128:
            jt = N // 128
            for r in range(N % 128, 128, 7):
                g, l = r // 16, r % 16
                assert P[pos(jt, 0, g, 0, l, 0)] == 0 and P[pos(jt, 0, g + 8, 1, 48 + l, 7)] == 0
        if K % 64:
            kk = K % 64
            for n in range(0, N, 37):
                r = n % 128
                assert P[pos(n // 128, KB - 1, r // 16, kk // 32, ((kk % 32) // 8) * 16 + r % 16, kk % 8)] == 0


# The five Qwen-2.5-shaped workloads, eight (workload, M) points.
POINTS = [(w.index, m) for w in inputs.WORKLOADS for m in w.ms]


def _points_id(p):
    return "%s-M%d" % (inputs.WORKLOADS[p[0]].name, p[1])


@pytest.mark.parametrize("point", POINTS, ids=[_points_id(p) for p in POINTS])
def test_integer_regime_bitwise_at_workload_shapes(dev, point):
    """Integer inputs: Gate/Up exact in any order, SiLU(Gate) == Gate, so every
    schedule must reproduce the whole oracle output bit for bit."""
    w = inputs.WORKLOADS[point[0]]
    M = point[1]
    A, W1, W2 = inputs.integer_case(M, w.K, w.N, seed=w.index * 10 + 1)
    outs = run_all_variants(dev, A, W1, W2, "int-" + _points_id(point))
    say("  oracle, all %d x %d elements" % (M, w.N))
    ref = cached_oracle("int-%s-M%d" % (w.name, M), lambda: oracle.swiglu(A, W1, W2))
    for name, y in outs.items():
        idx = diff_positions(y, ref)
        assert idx.size == 0, "%s: %d of %d elements differ bitwise from the oracle, first at %s" % (
            name, idx.size, ref.size, list(map(int, np.unravel_index(int(idx[0]), ref.shape))))


@pytest.mark.parametrize("point", POINTS, ids=[_points_id(p) for p in POINTS])
def test_gaussian_workloads(dev, point):
    """Seeded N(0,1) activations, N(0,1/K) weights at the workload shapes:
    every element of every schedule against the whole oracle output, with the
    bitwise and the pages' > 1 % mismatch rates over all elements."""
    w = inputs.WORKLOADS[point[0]]
    M = point[1]
    A, W1, W2 = inputs.workload_tensors(w, M)
    outs = run_all_variants(dev, A, W1, W2, "gauss-" + _points_id(point))
    say("  oracle, all %d x %d elements" % (M, w.N))
    ref, P = cached_oracle("gauss-%s-M%d" % (w.name, M), lambda: oracle.swiglu(A, W1, W2, want_p=True),
                           want_p=True)
    metric = PageMetric(ref, P)
    say("  oracle's own bf16 vs its fp32: >1%% rel err %.5f%%" % (100 * metric.base_count / max(1, ref.size)))
    for name, y in outs.items():
        idx = check_close_all(y, ref, name)
        b, pg = metric.rates(idx, y)
        say("  %s: all %d elements within tolerance; bitwise mismatch %.5f%%, >1%% rel err vs fp32 %.5f%%"
            % (name, ref.size, 100 * b, 100 * pg))


@pytest.mark.parametrize("tail", [False, True], ids=["no-tail", "mixed-tail"])
def test_persistent_multi_tile_walk(dev, tail):
    """Persistent 256-row tiles, each workgroup walking several of them: the
    next tile's stages issued during the epilogue, the Y stores left in flight
    into the next K loop, the accumulators and read bases reset per tile.
    M = 4096 (16 row tiles) and N from the device's CU count, so the tile
    count is four per CU (no tail) or four per CU plus 128 tiles that run as
    the mixed launch's 128-row tail; ragged K (136 = 2 x 64 + 8).  Every
    element of every schedule against the oracle."""
    cus = sw.swiglu_device_cu_count()
    cols = max(4, cus // 4) + (8 if tail else 0)
    M, K, N = 4096, 136, 128 * cols
    tiles = (M // 256) * cols
    assert tiles >= 3 * cus, "shape does not make each workgroup walk several tiles"
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=M + 5 * K + N)
    outs = run_all_variants(dev, A, W1, W2, "walk")
    ref = oracle.swiglu(A, W1, W2)
    for name, y in outs.items():
        check_close_all(y, ref, "walk/%s %s" % (name, (M, K, N)))
    assert np.array_equal(outs["fused"], outs["dp"]), "fused != fused_packed(dp) bitwise"


def test_unfused_pipeline(dev):
    M, K, N = 64, 896, 4864
    A, W1, W2 = inputs.workload_tensors(inputs.WORKLOADS[0])
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    G, U, Y = sw.swiglu_unfused(Ad, W1d, W2d)
    torch.cuda.synchronize()
    Gb, Ub, Yb = gpu_bits(G), gpu_bits(U), gpu_bits(Y)
    # each GEMM: the fp32 sums differ only in order, so bf16 results are within 1 ulp
    # (plus an absolute floor for sums that cancel to near zero)
    for name, got, w in (("G", Gb, W1), ("U", Ub, W2)):
        ref = oracle.gemm_bf16(A, w)
        g, r = f32(got).astype(np.float64), f32(ref).astype(np.float64)
        bad = np.argwhere(np.abs(g - r) > 2.0 ** -7 * np.abs(r) + 1e-3)
        assert bad.size == 0, "%s: %d elements beyond 1 ulp, e.g. %s got %r want %r" % (
            name, len(bad), bad[0].tolist(), g[tuple(bad[0])], r[tuple(bad[0])])
    # the element-wise step on the GPU's own G and U
    check_close(Yb, oracle.silu_mul(Gb, Ub), "silu_mul")
    # the whole pipeline against the oracle's fused result: double rounding of
    # Gate and Up adds error, report it
    ref, P = oracle.swiglu(A, W1, W2, want_p=True)
    b, pg = mismatch_rates(Yb, ref, P)
    say("  unfused vs fused oracle: bitwise mismatch %.4f%%, >1%% rel err %.4f%%" % (100 * b, 100 * pg))
    # stand-alone silu_mul with an odd count (vector body + scalar tail)
    cnt = 1000003
    g = torch.randn(cnt, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    u = torch.randn(cnt, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    y = sw.swiglu_silu_mul(g.to(dev), u.to(dev))
    torch.cuda.synchronize()
    check_close(gpu_bits(y), oracle.silu_mul(inputs.as_bits(g), inputs.as_bits(u)), "silu_mul odd")


def test_invariants_at_decode_shape(dev):
    K, N = 3584, 18944
    A, W1, W2 = inputs.workload_tensors(inputs.WORKLOADS[2], 16)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    Wp = sw.swiglu_pack_weights(W1d, W2d)
    for v in (DP, SPLIT, DECODE):
        base = sw.swiglu_fused_packed(Ad, Wp, N, variant=v)
        again = sw.swiglu_fused_packed(Ad, Wp, N, variant=v)
        torch.cuda.synchronize()
        assert torch.equal(base.view(torch.int16), again.view(torch.int16)), "not deterministic"
        # W1 = 0 -> Y = 0
        Z = sw.swiglu_pack_weights(torch.zeros_like(W1d), W2d)
        assert torch.all(sw.swiglu_fused_packed(Ad, Z, N, variant=v).float() == 0)
        # zero W2 column -> zero Y column, others unchanged
        W2z = W2d.clone()
        W2z[:, 777] = 0
        Yz = sw.swiglu_fused_packed(Ad, sw.swiglu_pack_weights(W1d, W2z), N, variant=v)
        assert torch.all(Yz[:, 777].float() == 0)
        keep = [c for c in range(N) if c != 777]
        assert torch.equal(Yz[:, keep].view(torch.int16), base[:, keep].view(torch.int16))
        # W2 -> 2 W2 doubles Y exactly
        Y2 = sw.swiglu_fused_packed(Ad, sw.swiglu_pack_weights(W1d, W2d * 2), N, variant=v)
        assert torch.equal(Y2.float(), 2 * base.float())
        # joint column permutation
        perm = torch.randperm(N, generator=torch.Generator().manual_seed(5)).to(dev)
        Yp = sw.swiglu_fused_packed(Ad, sw.swiglu_pack_weights(W1d[:, perm].contiguous(),
                                                               W2d[:, perm].contiguous()), N, variant=v)
        assert torch.equal(Yp.view(torch.int16), base[:, perm].view(torch.int16))
        # swapping Gate and Up changes the result
        Ys = sw.swiglu_fused_packed(Ad, sw.swiglu_pack_weights(W2d, W1d), N, variant=v)
        assert not torch.equal(Ys.view(torch.int16), base.view(torch.int16))
    # one-hot rows select weight rows: Gate = W1[k], Up = W2[k] exactly
    Ah = A.clone()
    ks = [0, 1234, 3583]
    for i, k in enumerate(ks):
        Ah[i] = 0
        Ah[i, k] = 1.0
    Yh = gpu_bits(sw.swiglu_fused_packed(Ah.to(dev), Wp, N))
    torch.cuda.synchronize()
    refh = oracle_rows(Ah, W1, W2, list(range(len(ks))))
    check_close(Yh[:len(ks)], refh, "one-hot rows")
    # prefix: the M=1 call equals row 0 of the M=16 call (same schedule class)
    Y1 = gpu_bits(sw.swiglu_fused_packed(Ad[:1].contiguous(), Wp, N))
    Y16 = gpu_bits(sw.swiglu_fused_packed(Ad, Wp, N))
    check_close(Y1, Y16[:1], "prefix M=1 vs M=16")


def test_edge_cases(dev):
    K, N = 128, 256
    A, W1, W2 = inputs.gaussian_case(5, K, N, seed=77)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    # M = 0
    y0 = sw.swiglu_fused(Ad[:0], W1d, W2d)
    assert y0.shape == (0, N)
    Wp = sw.swiglu_pack_weights(W1d, W2d)
    assert sw.swiglu_fused_packed(Ad[:0], Wp, N).shape == (0, N)
    # W1 == W2 is legal: Y = SiLU(G) * G
    ys = gpu_bits(sw.swiglu_fused(Ad, W1d, W1d))
    check_close(ys, oracle.swiglu(A, W1, W1), "W1 == W2")
    # misaligned operand is rejected before launch
    buf = torch.empty(5 * K + 1, dtype=torch.bfloat16, device=dev)
    Amis = buf[1:].view(5, K)
    with pytest.raises(sw.SwigluError) as ei:
        sw.swiglu_fused(Amis, W1d, W2d)
    assert ei.value.status == 4
    # overflow regime: Gate <= -K -> SiLU = -0 -> Y = +-0
    A2, W12, W22 = inputs.integer_case(64, 896, 512, seed=3, w1_vals=(-3, -2, -1))
    Y = sw.swiglu_fused(A2.to(dev), W12.to(dev), W22.to(dev))
    torch.cuda.synchronize()
    assert np.all((gpu_bits(Y) & 0x7FFF) == 0)


@pytest.mark.parametrize("M,K,N", [
    (16, 136, 520),       # decode schedule
    (100, 136, 520),      # panel schedule
    (300, 136, 1032),     # 128-row tiles
    (2100, 72, 264),      # persistent 256-row tiles with the 128-row tail
])
def test_nonfinite_inputs(dev, M, K, N):
    """IEEE special values pass through every schedule as the oracle's
    definition gives them: a NaN activation makes its whole output row NaN;
    +Inf in a row gives Gate and Up of +-Inf (SiLU(+Inf) = +Inf, and
    SiLU(-Inf) = -Inf / Inf = NaN); an Inf weight does the same to its output
    column.  The NaN pattern must match exactly, and finite and infinite values
    as everywhere (the last activation K column, in the ragged block, too)."""
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=M + 11 * K + N)
    nan, inf = float("nan"), float("inf")
    A[1, 5] = nan
    A[2, 7] = inf
    A[3, 9] = -inf
    A[M - 1, K - 1] = nan
    W1[3, 10] = inf
    W2[K - 1, N - 2] = -inf
    outs = run_all_variants(dev, A, W1, W2, "nonfinite")
    ref = oracle.swiglu(A, W1, W2)
    r = f32(ref)
    assert np.isnan(r[1]).all() and np.isnan(r[M - 1]).all() and np.isinf(r[2]).any()
    for name, y in outs.items():
        check_close(y, ref, "nonfinite/%s %s" % (name, (M, K, N)))


@pytest.mark.parametrize("M,K,N,auto_decode", [
    (1, 6144, 24576, True),    # long K, >= 192 column tiles: 8 column groups per workgroup
    (16, 3584, 4096, True),    # short K: one column group, 8 K blocks in flight, activations via LDS
    (8, 1000, 2056, True),     # the same with at most 8 rows: activations from global, ragged K
    (32, 6144, 12288, True),   # long K, M <= 32, under two workgroups per CU: 4 column groups
    (32, 512, 16384, True),    # M <= 32, wide N: 8 column groups
    (24, 512, 4096, True),     # M <= 32, short K, narrow N: 2 column groups, 2 K blocks in flight
    (48, 6144, 12288, False),  # long K, M <= 64: 4 column groups (AUTO takes the panel schedule)
    (64, 1024, 2048, True),    # short K, M <= 64, few panels: 2 column groups, activations via LDS
])
def test_decode_configurations(dev, M, K, N, auto_decode):
    """Every decode configuration by M, K and N (column groups per workgroup,
    K blocks in flight) against the oracle, all rows; AUTO picks decode for
    the shapes it should."""
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=M + K + N)
    Wp = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    Y = sw.swiglu_fused_packed(A.to(dev), Wp, N, variant=DECODE)
    Ya = sw.swiglu_fused_packed(A.to(dev), Wp, N, variant=AUTO)
    torch.cuda.synchronize()
    assert (sw.swiglu_choose_variant(M, K, N) == DECODE) == auto_decode
    ref = oracle.swiglu(A, W1, W2)
    check_close(gpu_bits(Y), ref, "decode %s" % ((M, K, N),))
    check_close(gpu_bits(Ya), ref, "auto %s" % ((M, K, N),))


@pytest.mark.parametrize("grid", ["one-per-cu", "narrow", "wide"])
@pytest.mark.parametrize("M,K", [(1, 136), (7, 72), (32, 200), (17, 1000), (33, 136), (64, 328)])
def test_rowmajor_decode_widths(dev, M, K, grid):
    """swiglu_fused at M <= 64 on each of its small-M schedules: the row-major
    decode kernel with 32-column workgroups (two K blocks in flight for one
    token tile, one for two) while 64-column ones would number under 1.5 per
    CU, with 64-column ones above that, and for 32 < M <= 64 with more
    32-column workgroups than CUs the 64x64 tile kernel; ragged K and a
    partial last workgroup of columns, every element against the oracle."""
    cus = sw.swiglu_device_cu_count()
    wide_min = 64 * ((3 * cus + 1) // 2)          # the narrowest N with 64-column workgroups
    N = {"one-per-cu": 32 * cus - 24, "narrow": wide_min - 64 * 3 - 24, "wide": wide_min + 40}[grid]
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=5 * M + K + N)
    say("[rowmajor decode] M=%d K=%d N=%d grid=%s" % (M, K, N, grid))
    Y = sw.swiglu_fused(A.to(dev), W1.to(dev), W2.to(dev))
    torch.cuda.synchronize()
    check_close(gpu_bits(Y), oracle.swiglu(A, W1, W2), "rowmajor decode %s" % ((M, K, N),))


@pytest.mark.parametrize("M,K,N", [
    (128, 200, 9000),     # 71 tiles of 128 columns: 141 of 64 columns, one round
    (100, 136, 30000),    # 235 tiles of 128 columns: 469 of 64 columns; M tail
    (300, 72, 8200),      # 3 x 65 tiles of 128 columns: 3 x 129 = 387 of 64 columns
    (130, 64, 18944),     # 2 x 148 tiles of 128 columns: one round of 148 256-row tiles instead
    (300, 136, 18944),    # 3 x 148 128-row tiles against 2 x 148 256-row ones: stays on 128 rows
    (450, 200, 30000),    # 2 x 235 256-row tiles (two rounds) against 4 x 235 128-row ones (four)
])
def test_rowmajor_prefill_tiles(dev, M, K, N):
    """swiglu_fused for 64 < M <= 512 on 128x64 tiles (when 128x128 tiles
    leave CUs idle and the 64-column grid fits one round or fills one and a
    half), on 128x128 tiles, and on 256x128 tiles where they need fewer rounds
    over the CUs by more than their 4/3 cost; ragged K and N, every element
    against the oracle."""
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=3 * M + K + N)
    say("[rowmajor prefill] M=%d K=%d N=%d" % (M, K, N))
    Y = sw.swiglu_fused(A.to(dev), W1.to(dev), W2.to(dev))
    torch.cuda.synchronize()
    check_close(gpu_bits(Y), oracle.swiglu(A, W1, W2), "rowmajor prefill %s" % ((M, K, N),))


@pytest.mark.parametrize("M,K,N", [
    # two rows of 128-row tiles on a wide product: one row of 256-row tiles on
    # the panel schedule (ragged K, partial last packed tile, M tail)
    (200, 136, 16392), (256, 72, 30000), (129, 64, 24576),
    (100, 256, 8192),     # 256 panels: one per workgroup
    (72, 64, 12040),      # one or two panels per workgroup; the last panel partly past N
    (128, 200, 24576),    # three panels per workgroup, across packed-tile borders; ragged K
    (96, 136, 30000),     # three or four panels; a partial last packed tile
])
def test_panel_schedule(dev, M, K, N):
    """One row of 128-row tiles (or, for two rows on a wide product, one row
    of 256-row tiles) with fewer column tiles than CUs: the 32-column weight
    panels are spread over the workgroups (data-parallel and AUTO), all
    elements against the oracle and bitwise against the row-major entry point
    (same MFMA chain per element)."""
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=M + 3 * K + N)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    Wp = sw.swiglu_pack_weights(W1d, W2d)
    say("[panels] M=%d K=%d N=%d" % (M, K, N))
    ys = {name: gpu_bits(sw.swiglu_fused_packed(Ad, Wp, N, variant=v)) for name, v in (("dp", DP), ("auto", AUTO))}
    yf = gpu_bits(sw.swiglu_fused(Ad, W1d, W2d))
    torch.cuda.synchronize()
    ref = oracle.swiglu(A, W1, W2)
    for name, y in ys.items():
        check_close(y, ref, "panels/%s %s" % (name, (M, K, N)))
        assert np.array_equal(y, yf), "panels/%s != fused bitwise" % name


@pytest.mark.parametrize("M,K,N", [
    (96, 256, 520),       # panel schedule, partial last packed tile
    (16, 3584, 18944),    # 7B decode width: decode schedule, long down-projection reduction
    (256, 896, 4864),     # 0.5B shape, a slice of the prefill rows
    (128, 1024, 6144),    # down projection split over K (4 column tiles for 256 CUs)
])
def test_mlp_block(dev, M, K, N):
    """The gated MLP block, fused and unfused: the fused Y against the
    oracle's SwiGLU product, the unfused Y against the oracle's element-wise
    step on the GPU's own bf16 Gate and Up (their one-ulp rounding
    differences from summation order are checked by test_unfused_pipeline),
    Z against the oracle's GEMM of the GPU's own Y (isolating the down
    projection, on the single-weight pack of W3), and the fused block's Y
    bitwise equal to a plain swiglu_fused_packed call."""
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=7 * M + K + N)
    W3 = inputs.weight(N, K, seed=M + K)
    Ad, W1d, W2d, W3d = A.to(dev), W1.to(dev), W2.to(dev), W3.to(dev)
    Wp = sw.swiglu_pack_weights(W1d, W2d)
    say("[mlp] M=%d K=%d N=%d" % (M, K, N))
    W3g = sw.swiglu_gemm_pack_weight(W3d)
    W1g, W2g = sw.swiglu_gemm_pack_weight(W1d), sw.swiglu_gemm_pack_weight(W2d)
    if (M, K, N) == (128, 1024, 6144):
        assert sw.swiglu_gemm_workspace_bytes(M, N, K) > 0, "down projection expected to take split-K"
    Yf, Zf = sw.swiglu_mlp_packed(Ad, Wp, W3g, N)
    G = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    U = torch.empty_like(G)
    Yu, Zu = sw.swiglu_mlp_unfused(Ad, W1g, W2g, W3g, N, G=G, U=U)
    Y0 = sw.swiglu_fused_packed(Ad, Wp, N)
    torch.cuda.synchronize()
    yf, zf, yu, zu = gpu_bits(Yf), gpu_bits(Zf), gpu_bits(Yu), gpu_bits(Zu)
    assert zf.shape == (M, K) and zu.shape == (M, K)
    assert np.array_equal(yf, gpu_bits(Y0)), "MLP's Y != swiglu_fused_packed bitwise"
    check_close(yf, oracle.swiglu(A, W1, W2), "mlp fused Y")
    check_close(yu, oracle.silu_mul(gpu_bits(G), gpu_bits(U)), "mlp unfused Y")
    check_gemm_ulp(gpu_bits(G), oracle.gemm_bf16(A, W1), "mlp unfused G")
    check_gemm_ulp(gpu_bits(U), oracle.gemm_bf16(A, W2), "mlp unfused U")
    W3b = inputs.as_bits(W3)
    check_gemm_ulp(zf, oracle.gemm_bf16(yf, W3b), "mlp fused Z")
    check_gemm_ulp(zu, oracle.gemm_bf16(yu, W3b), "mlp unfused Z")
    Zd = sw.swiglu_mlp_down(Yf, W3g, K)
    torch.cuda.synchronize()
    check_gemm_ulp(gpu_bits(Zd), oracle.gemm_bf16(yf, W3b), "mlp down projection alone")


def test_interleaved_pack_roundtrip_and_layout(dev):
    """Column-granular interleaved pack: unpack(pack(W)) == W bitwise, packed
    row 2c of a tile holds W1 column c and row 2c + 1 holds W2 column c, and
    the padding (columns past N, k past K) is zero."""
    for K, N in [(64, 128), (72, 136), (200, 520)]:
        _, W1, W2 = inputs.gaussian_case(1, K, N, seed=3 * K + N)
        W1d, W2d = W1.to(dev), W2.to(dev)
        Wp = sw.swiglu_pack_weights_interleaved(W1d, W2d)
        V1, V2 = sw.swiglu_unpack_weights_interleaved(Wp, K, N)
        torch.cuda.synchronize()
        assert torch.equal(V1.view(torch.int16), W1d.view(torch.int16))
        assert torch.equal(V2.view(torch.int16), W2d.view(torch.int16))
        P = inputs.as_bits(Wp.cpu())
        KB = (K + 63) // 64
        w1, w2 = inputs.as_bits(W1), inputs.as_bits(W2)

        def pos(jt, kb, prow, k):
            g, r, h, kk = prow // 16, prow % 16, k // 32, k % 32
            return ((((jt * KB + kb) * 16 + g) * 2 + h) * 64 + (kk // 8) * 16 + r) * 8 + kk % 8

        for n in range(0, N, 3):
            for k in range(0, K, 5):
                jt, c = n // 128, n % 128
                assert P[pos(jt, k // 64, 2 * c, k % 64)] == w1[k, n]
                assert P[pos(jt, k // 64, 2 * c + 1, k % 64)] == w2[k, n]
        JT = (N + 127) // 128
        for c in range(N % 128 or 128, 128):
            for k in range(0, 64, 9):
                assert P[pos(JT - 1, 0, 2 * c, k)] == 0 and P[pos(JT - 1, 0, 2 * c + 1, k)] == 0
        if K % 64:
            for n in range(0, N, 11):
                for k in range(K % 64, 64, 5):
                    assert P[pos(n // 128, KB - 1, 2 * (n % 128), k)] == 0


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 128), (40, 200, 520), (128, 512, 4096), (300, 136, 264),
    (2100, 72, 256), (4000, 200, 2696),
    (200, 136, 16392),    # one row of 256-row tiles on the panel schedule
])
def test_interleaved_layout_matches(dev, M, K, N):
    """The interleaved-layout path against the oracle and bitwise against the
    per-tile layout on the same schedule (one decode-sized M, panel schedule,
    128-row tiles, 256-row tiles with the mixed tail; ragged K and N)."""
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=5 * M + K + N)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    say("[interleaved] M=%d K=%d N=%d" % (M, K, N))
    Wi = sw.swiglu_pack_weights_interleaved(W1d, W2d)
    Yi = gpu_bits(sw.swiglu_fused_packed_interleaved(Ad, Wi, N))
    check_close(Yi, oracle.swiglu(A, W1, W2), "interleaved %s" % ((M, K, N),))
    if M > 64:
        Wp = sw.swiglu_pack_weights(W1d, W2d)
        Yp = gpu_bits(sw.swiglu_fused_packed(Ad, Wp, N, variant=DP))
        assert np.array_equal(Yi, Yp), "interleaved != per-tile layout bitwise"


@pytest.mark.parametrize("point", POINTS, ids=[_points_id(p) for p in POINTS])
def test_interleaved_workload_shapes(dev, point):
    """The interleaved-layout path at the workload points: every element
    against the whole oracle output (the same inputs and cached result as
    test_gaussian_workloads), and bitwise equal to the per-tile layout on the
    same streaming schedule."""
    w = inputs.WORKLOADS[point[0]]
    M = point[1]
    A, W1, W2 = inputs.workload_tensors(w, M)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    say("[interleaved-workload] %s M=%d" % (w.name, M))
    Yi = gpu_bits(sw.swiglu_fused_packed_interleaved(Ad, sw.swiglu_pack_weights_interleaved(W1d, W2d), w.N))
    Yp = gpu_bits(sw.swiglu_fused_packed(Ad, sw.swiglu_pack_weights(W1d, W2d), w.N, variant=DP))
    ref, _ = cached_oracle("gauss-%s-M%d" % (w.name, M), lambda: oracle.swiglu(A, W1, W2, want_p=True),
                           want_p=True)
    check_close_all(Yi, ref, "interleaved %s M=%d" % (w.name, M))
    assert np.array_equal(Yi, Yp), "interleaved != per-tile layout bitwise"


def test_split_workspace_reused_across_shapes(dev):
    """One workspace serves split-K calls of different shapes in a row, and
    its earlier contents (partials of another shape, or garbage) never leak
    into a result."""
    ws = sw.Workspace(dev)
    shapes = [(128, 2048, 1024), (128, 2048, 18944), (128, 1024, 4864), (128, 2048, 18944), (96, 512, 8192)]
    for i, (M, K, N) in enumerate(shapes):
        A, W1, W2 = inputs.gaussian_case(M, K, N, seed=300 + i)
        Wp = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
        Y = sw.swiglu_fused_packed(A.to(dev), Wp, N, workspace=ws, variant=SPLIT)
        torch.cuda.synchronize()
        rows = sample_rows(M, 4)
        check_close(gpu_bits(Y)[rows], oracle_rows(A, W1, W2, rows), "split reuse %s" % ((M, K, N),))
        ws.buf.fill_(0x7F)      # NaN-patterned leftovers must not matter to the next call


def test_split_workspace_grows_on_call_stream(dev):
    """Split-K calls queued on a stream other than the current one, each
    needing a larger workspace than the last: the grown buffer is allocated
    on the calls' stream, so the memory of the buffer it replaces is not
    handed to the current stream's allocations (filled meanwhile) while the
    earlier calls still write their partial sums into it."""
    side = torch.cuda.Stream()
    ws = sw.Workspace(dev)
    cases = []
    for i, (M, K, N) in enumerate([(128, 1024, 1024), (128, 2048, 4864), (128, 2048, 18944)]):
        A, W1, W2 = inputs.gaussian_case(M, K, N, seed=400 + i)
        cases.append((A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev)), N))
    torch.cuda.synchronize()
    say("[side stream] split-K with a growing workspace")
    outs, junk = [], []
    for Ad, Wp, N in cases:
        outs.append(sw.swiglu_fused_packed(Ad, Wp, N, workspace=ws, variant=SPLIT, stream=side))
        junk.append(torch.full((4 << 20,), 0x7F, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    for (Ad, Wp, N), Y in zip(cases, outs):
        ref = sw.swiglu_fused_packed(Ad, Wp, N, variant=SPLIT)
        torch.cuda.synchronize()
        assert np.array_equal(gpu_bits(Y), gpu_bits(ref)), "side-stream split-K call differs (N=%d)" % N


@pytest.mark.parametrize("M,K,N", [(1, 200, 264), (17, 136, 520), (32, 896, 4864), (33, 72, 264),
                                   (48, 200, 1032), (64, 896, 4864),
                                   (65, 72, 264), (300, 200, 520), (1024, 896, 4864), (2100, 136, 256),
                                   (4096, 896, 4864)])
def test_gemm_bf16_against_oracle(dev, M, K, N):
    """The unfused pipeline's GEMM: bf16 of an fp32 sum, so the GPU and the
    oracle differ by at most one bf16 rounding flip of sums that differ only in
    order (plus an absolute floor for sums that cancel to near zero)."""
    A, W, _ = inputs.gaussian_case(M, K, N, seed=M + K)
    C = sw.swiglu_gemm_bf16(A.to(dev), W.to(dev))
    torch.cuda.synchronize()
    check_gemm_ulp(gpu_bits(C), oracle.gemm_bf16(A, W), "gemm %s" % ((M, K, N),))


def check_gemm_ulp(got_bits, ref_bits, what):
    """A bf16 GEMM result: every element within one bf16 rounding flip of the
    oracle's (fp32 sums that differ only in order), plus an absolute floor for
    sums that cancel to near zero."""
    got = f32(got_bits).astype(np.float64)
    ref = f32(ref_bits).astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    bad = np.argwhere(np.abs(got - ref) > 2.0 ** -7 * np.abs(ref) + 1e-3)
    assert bad.size == 0, "%s: %d elements beyond 1 ulp, e.g. %s got %r want %r" % (
        what, len(bad), bad[0].tolist(), got[tuple(bad[0])], ref[tuple(bad[0])])


@pytest.mark.parametrize("M,K,N", [
    # decode GEMM, each of its configurations on a 256-CU chip:
    (1, 200, 264),                  # <1,1,14> on weight halves (M <= 8)
    (16, 3584, 1032),               # <1,1,8> on halves, activations via LDS
    (12, 200, 16400),               # the same, wide, ragged K
    (3, 6200, 16400),               # <1,4,4> on halves (long K, wide)
    (17, 136, 520), (32, 896, 4864),  # <2,2,2>
    (24, 6200, 24600),              # <2,8,1> on halves (long K, wide)
    (20, 6200, 1000),               # <2,2,2> on halves (long K, narrow)
    (48, 200, 1032), (64, 72, 136),   # <4,1,1> on halves, activations via LDS (short, ragged K)
    (40, 2104, 520),                # the same, 33 K blocks
    (64, 3584, 18944),                                                     # panel schedule: half-panels
    (72, 200, 30584),                                                      # 3-4 half-panels per workgroup
    (128, 4864, 896),                                                      # down-projection shape: 3.5 tiles
    (300, 200, 520), (2100, 136, 264),                                     # 128-row tiles
    (2304, 128, 7680),                                                     # 256-row tiles + 128-row tail
    (4096, 136, 16384),                                                    # four 256-row tiles per workgroup
])
def test_gemm_packed_against_oracle(dev, M, K, N):
    """The plain GEMM on the single-weight pack, through every schedule of the
    fused product (decode, panels, 128-row tiles, persistent 256-row tiles
    with the mixed tail): every element within one bf16 rounding flip of the
    oracle's GEMM; partial last tiles in both halves (N not a multiple of 256
    or of 128), ragged K."""
    A, W, _ = inputs.gaussian_case(M, K, N, seed=3 * M + K + 7 * N)
    say("[gemm_packed] M=%d K=%d N=%d" % (M, K, N))
    Wg = sw.swiglu_gemm_pack_weight(W.to(dev))
    C = sw.swiglu_gemm_packed(A.to(dev), Wg, N)
    torch.cuda.synchronize()
    check_gemm_ulp(gpu_bits(C), oracle.gemm_bf16(A, W), "gemm_packed %s" % ((M, K, N),))


@pytest.mark.parametrize("M,K,N", [
    (128, 4864, 896),     # 0.5B down-projection width: 4 column tiles, 2 splits
    (100, 6200, 1000),    # ragged M, K and N (half-empty last packed tile), 3 splits
    (1100, 1000, 520),    # compute-bound, 27 data-parallel tiles: split anyway, 8 splits
])
def test_gemm_split_k(dev, M, K, N):
    """The GEMM's split-K schedule (taken only with a workspace that holds
    the partial sums): every element within one bf16 flip of the oracle, the
    same as the data-parallel schedule up to that flip, and bitwise
    repeatable with a workspace full of NaN or of the previous call's
    partials."""
    need = sw.swiglu_gemm_workspace_bytes(M, K, N)
    assert need > 0, "shape expected to take split-K"
    A, W, _ = inputs.gaussian_case(M, K, N, seed=5 * M + K + 3 * N)
    say("[gemm_split] M=%d K=%d N=%d need=%d" % (M, K, N, need))
    Ad, Wg = A.to(dev), sw.swiglu_gemm_pack_weight(W.to(dev))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    C1 = sw.swiglu_gemm_packed(Ad, Wg, N, workspace=ws)
    C2 = sw.swiglu_gemm_packed(Ad, Wg, N, workspace=ws)
    C0 = sw.swiglu_gemm_packed(Ad, Wg, N, workspace=torch.empty(16, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    ref = oracle.gemm_bf16(A, W)
    check_gemm_ulp(gpu_bits(C1), ref, "gemm split-K %s" % ((M, K, N),))
    check_gemm_ulp(gpu_bits(C0), ref, "gemm data-parallel %s" % ((M, K, N),))
    assert np.array_equal(gpu_bits(C1), gpu_bits(C2)), "split-K GEMM not repeatable"


def test_gemm_pack_layout(dev):
    """Single-weight pack as documented in swiglu.h: tile jt holds columns
    jt*256 + g*16 + l%16 in 16-row group g; padding (columns past N, k past
    K) is zero."""
    for K, N in [(64, 256), (72, 264), (200, 1032)]:
        _, W, _ = inputs.gaussian_case(1, K, N, seed=5 * K + N)
        P = inputs.as_bits(sw.swiglu_gemm_pack_weight(W.to(dev)).cpu())
        assert P.size * 2 == sw.swiglu_gemm_packed_bytes(K, N)
        w = inputs.as_bits(W)
        KB, JT = (K + 63) // 64, (N + 255) // 256

        def pos(jt, kb, g, h, l, e):
            return ((((jt * KB + kb) * 16 + g) * 2 + h) * 64 + l) * 8 + e

        for n in range(0, N, 3):
            for k in range(0, K, 7):
                jt, r, kb, kk = n // 256, n % 256, k // 64, k % 64
                g, h, l, e = r // 16, kk // 32, ((kk % 32) // 8) * 16 + r % 16, kk % 8
                assert P[pos(jt, kb, g, h, l, e)] == w[k, n]
        for r in range(N % 256 or 256, 256):
            assert P[pos(JT - 1, 0, r // 16, 0, r % 16, 0)] == 0
        if K % 64:
            for n in range(0, N, 13):
                r, kk = n % 256, K % 64
                assert P[pos(n // 256, KB - 1, r // 16, kk // 32, ((kk % 32) // 8) * 16 + r % 16, kk % 8)] == 0


@pytest.mark.parametrize("M,K,N", [(16, 3584, 18944), (64, 896, 4864), (4096, 896, 4864)])
def test_unfused_packed_pipeline(dev, M, K, N):
    """The unfused pipeline on the packed GEMM: G and U within one bf16 flip
    of the oracle's GEMMs, Y within tolerance of the oracle's element-wise
    step on the GPU's own G and U."""
    A, W1, W2 = inputs.gaussian_case(M, K, N, seed=M + 2 * K + N)
    Ad = A.to(dev)
    W1g, W2g = sw.swiglu_gemm_pack_weight(W1.to(dev)), sw.swiglu_gemm_pack_weight(W2.to(dev))
    say("[unfused_packed] M=%d K=%d N=%d" % (M, K, N))
    G, U, Y = sw.swiglu_unfused_packed(Ad, W1g, W2g, N)
    torch.cuda.synchronize()
    Gb, Ub, Yb = gpu_bits(G), gpu_bits(U), gpu_bits(Y)
    rows = list(range(M)) if M <= 64 else sample_rows(M, 16)
    check_gemm_ulp(Gb[rows], oracle.gemm_bf16(A[rows].contiguous(), W1), "G")
    check_gemm_ulp(Ub[rows], oracle.gemm_bf16(A[rows].contiguous(), W2), "U")
    check_close(Yb, oracle.silu_mul(Gb, Ub), "silu_mul of the GPU's own G, U")
