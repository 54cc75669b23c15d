"""The C ABI without a GPU: the library loads, exports every entry point that
include/swiglu.h declares, and rejects bad arguments on the host before any
HIP call (so these calls are safe on a machine with no device)."""
import ctypes
import os
import re

import pytest

import swiglu_gated_mlp_amd as sw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("swiglu.h", "swiglu_probe.h")]

OK, NULLP, SHAPE, UNSUP, MISAL, ALIAS, WS, VARIANT = 0, 1, 2, 3, 4, 5, 6, 7


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swiglu_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_set():
    assert set(declared_functions()) == set(sw.SIGNATURES), \
        "header and binding disagree: %s" % (set(declared_functions()) ^ set(sw.SIGNATURES))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sw.LIB_PATH)
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, "not exported: %s" % missing


def test_abi_version_and_status_strings():
    assert sw.swiglu_abi_version() == 3
    for s in range(9):
        assert sw.status_str(s) and sw.status_str(s) != "unknown status"
    assert sw.status_str(99) == "unknown status"


def test_packed_bytes():
    L = sw.lib()
    # ceil(N/128) tiles x ceil(K/64) blocks x 256 rows x 64 k x 2 bytes
    assert L.swiglu_packed_bytes(896, 4864) == 38 * 14 * 256 * 64 * 2
    assert L.swiglu_packed_bytes(896, 4864) == 2 * 896 * 4864 * 2   # exact when tiles divide
    assert L.swiglu_packed_bytes(72, 136) == 2 * 2 * 256 * 64 * 2   # padded tail tiles
    assert L.swiglu_packed_bytes(8192, 29568) == 968884224
    assert L.swiglu_packed_bytes(0, 8) == 0 and L.swiglu_packed_bytes(12, 8) == 0


# fake, never-dereferenced device addresses: validation returns before any use
A_, W1_, W2_, Y_, WP_, WS_ = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000


@pytest.mark.parametrize("M,K,N,want", [
    (-1, 64, 64, SHAPE), (4, 0, 64, SHAPE), (4, 64, 0, SHAPE), (4, -8, 64, SHAPE),
    (4, 60, 64, UNSUP), (4, 64, 60, UNSUP), (1 << 31, 64, 64, SHAPE), (4, (1 << 22) + 8, 8, UNSUP),
])
def test_fused_shape_errors(M, K, N, want):
    assert sw.lib().swiglu_fused(A_, W1_, W2_, Y_, M, K, N, None) == want


def test_fused_pointer_errors():
    L = sw.lib()
    assert L.swiglu_fused(None, W1_, W2_, Y_, 4, 64, 64, None) == NULLP
    assert L.swiglu_fused(A_, W1_, W2_, None, 4, 64, 64, None) == NULLP
    assert L.swiglu_fused(A_ + 2, W1_, W2_, Y_, 4, 64, 64, None) == MISAL
    assert L.swiglu_fused(A_, W1_, W2_, Y_ + 8, 4, 64, 64, None) == MISAL
    # Y overlapping A, W1 or W2
    assert L.swiglu_fused(A_, W1_, W2_, A_ + 64, 4, 64, 64, None) == ALIAS
    assert L.swiglu_fused(A_, W1_, W2_, W2_ + 1024, 4, 64, 64, None) == ALIAS
    # W1 == W2 is allowed (inputs may alias): validation passes; M == 0 then returns OK
    assert L.swiglu_fused(A_, W1_, W1_, Y_, 0, 64, 64, None) == OK
    # M == 0 is a valid empty call even with null pointers
    assert L.swiglu_fused(None, None, None, None, 0, 64, 64, None) == OK


def test_packed_errors():
    L = sw.lib()
    assert L.swiglu_fused_packed(A_, WP_, Y_, 4, 64, 64, None, 0, 9, None) == VARIANT
    # the decode schedule serves M <= 64 only
    assert L.swiglu_fused_packed(A_, WP_, Y_, 65, 64, 64, None, 0, 3, None) == VARIANT
    assert L.swiglu_workspace_bytes(16, 3584, 18944, 3) == 0
    # the sequential order: any M, no workspace; codes past it are unknown
    assert L.swiglu_workspace_bytes(16, 3584, 18944, 4) == 0
    assert L.swiglu_workspace_bytes(8192, 3584, 18944, 4) == 0
    assert L.swiglu_fused_packed(A_, WP_, Y_, 4, 64, 64, None, 0, 5, None) == VARIANT
    assert L.swiglu_fused_packed(A_, None, Y_, 4, 64, 64, None, 0, 4, None) == NULLP
    assert L.swiglu_fused_packed(A_, WP_, Y_, 4, 64, 64, None, 0, -1, None) == VARIANT
    assert L.swiglu_fused_packed(A_, None, Y_, 4, 64, 64, None, 0, 0, None) == NULLP
    assert L.swiglu_fused_packed(A_, WP_, WP_ + 16, 4, 64, 64, None, 0, 1, None) == ALIAS
    # split-K needs a workspace
    need = L.swiglu_workspace_bytes(4, 4096, 1024, 2)
    assert need > 0
    assert L.swiglu_fused_packed(A_, WP_, Y_, 4, 4096, 1024, None, 0, 2, None) == WS
    assert L.swiglu_fused_packed(A_, WP_, Y_, 4, 4096, 1024, WS_, need - 1, 2, None) == WS
    assert L.swiglu_fused_packed(A_, WP_, Y_, 4, 4096, 1024, WS_ + 4, need, 2, None) == MISAL
    assert L.swiglu_fused_packed(A_, WP_, Y_, 4, 4096, 1024, Y_, need, 2, None) == ALIAS
    # the data-parallel schedule needs none
    assert L.swiglu_workspace_bytes(4, 4096, 1024, 1) == 0
    assert L.swiglu_pack_weights(W1_, W2_, W1_ + 16, 64, 64, None) == ALIAS
    assert L.swiglu_pack_weights(W1_, W2_, WP_, 63, 64, None) == UNSUP
    assert L.swiglu_unpack_weights(WP_, W1_, W1_, 64, 64, None) == ALIAS


def test_unfused_errors():
    L = sw.lib()
    assert L.swiglu_silu_mul(A_, W1_, Y_, -1, None) == SHAPE
    assert L.swiglu_silu_mul(A_, W1_, A_, 16, None) == ALIAS
    assert L.swiglu_silu_mul(None, None, None, 0, None) == OK
    assert L.swiglu_gemm_bf16(A_, W1_, A_ + 16, 4, 64, 64, None) == ALIAS
    assert L.swiglu_unfused(A_, W1_, W2_, Y_, Y_, WS_, 4, 64, 64, None) == ALIAS
    assert L.swiglu_unfused(A_, W1_, W2_, None, WP_, WS_, 4, 64, 64, None) == NULLP


Z_, W3_ = 0x70000000, 0x80000000


def test_mlp_errors():
    L = sw.lib()
    P = L.swiglu_mlp_packed
    # shapes, variants and the empty call come first
    assert P(A_, WP_, W3_, Y_, Z_, 4, 60, 64, None, 0, 0, None) == UNSUP
    assert P(A_, WP_, W3_, Y_, Z_, 4, 64, 64, None, 0, 9, None) == VARIANT
    assert P(None, None, None, None, None, 0, 64, 64, None, 0, 0, None) == OK
    # the down projection's own operands
    assert P(A_, WP_, None, Y_, Z_, 4, 64, 64, None, 0, 0, None) == NULLP
    assert P(A_, WP_, W3_, Y_, None, 4, 64, 64, None, 0, 0, None) == NULLP
    assert P(A_, WP_, W3_ + 8, Y_, Z_, 4, 64, 64, None, 0, 0, None) == MISAL
    assert P(A_, WP_, W3_, Y_, Z_ + 2, 4, 64, 64, None, 0, 0, None) == MISAL
    # Z [4, 64] overlapping A, W3 or Y; Y overlapping W3
    assert P(A_, WP_, W3_, Y_, A_ + 256, 4, 64, 64, None, 0, 0, None) == ALIAS
    assert P(A_, WP_, W3_, Y_, W3_ + 16, 4, 64, 64, None, 0, 0, None) == ALIAS
    assert P(A_, WP_, W3_, Y_, Y_ + 64, 4, 64, 64, None, 0, 0, None) == ALIAS
    assert P(A_, WP_, W3_, W3_ + 4096, Z_, 4, 64, 64, None, 0, 0, None) == ALIAS
    D = L.swiglu_mlp_down
    assert D(Y_, W3_, Z_, 4, 64, 60, None, 0, None) == UNSUP
    assert D(None, None, None, 0, 64, 64, None, 0, None) == OK
    assert D(Y_, None, Z_, 4, 64, 64, None, 0, None) == NULLP
    assert D(Y_ + 2, W3_, Z_, 4, 64, 64, None, 0, None) == MISAL
    assert D(Y_, W3_, Y_ + 128, 4, 64, 64, None, 0, None) == ALIAS
    assert D(Y_, W3_, W3_ + 16, 4, 64, 64, None, 0, None) == ALIAS
    U = L.swiglu_mlp_unfused
    G_, U_ = 0x90000000, 0xA0000000
    assert U(A_, W1_, W2_, W3_, G_, U_, Y_, Z_, 4, 64, 60, None, 0, None) == UNSUP
    assert U(None, None, None, None, None, None, None, None, 0, 64, 64, None, 0, None) == OK
    assert U(A_, W1_, W2_, W3_, G_, U_, Y_, None, 4, 64, 64, None, 0, None) == NULLP
    assert U(A_, W1_, W2_, W3_, G_, U_, Y_, Z_ + 4, 4, 64, 64, None, 0, None) == MISAL
    assert U(A_, W1_, W2_, W3_, G_, U_, Y_, G_ + 32, 4, 64, 64, None, 0, None) == ALIAS
    assert U(A_, W1_, W2_, W3_, G_, W3_ + 128, Y_, Z_, 4, 64, 64, None, 0, None) == ALIAS
    assert U(A_, W1_, W2_, W3_, G_, U_, Y_, Z_, 4, 64, 64, Z_ + 64, 256, None) == ALIAS


def test_gemm_packed_sizes_and_errors():
    """The single-weight pack: ceil(N/256) tiles of 256 packed rows, the fused
    pack's 32 KiB blocks per 64 k; the packed GEMM's validation codes."""
    L = sw.lib()
    assert L.swiglu_gemm_packed_bytes(896, 4864) == 19 * 14 * 256 * 64 * 2 == 896 * 4864 * 2
    assert L.swiglu_gemm_packed_bytes(8192, 29568) == 116 * 128 * 32768    # 115.5 tiles -> 116
    assert L.swiglu_gemm_packed_bytes(72, 136) == 1 * 2 * 32768
    assert L.swiglu_gemm_packed_bytes(12, 8) == 0 and L.swiglu_gemm_packed_bytes(8, 0) == 0
    G = L.swiglu_gemm_packed
    assert G(None, None, None, 0, 64, 64, None, 0, None) == OK
    assert G(A_, WP_, Y_, 4, 60, 64, None, 0, None) == UNSUP
    assert G(A_, None, Y_, 4, 64, 64, None, 0, None) == NULLP
    assert G(A_, WP_, Y_ + 2, 4, 64, 64, None, 0, None) == MISAL
    assert G(A_, WP_, WP_ + 1024, 4, 64, 64, None, 0, None) == ALIAS
    assert G(A_, WP_, A_ + 16, 4, 64, 64, None, 0, None) == ALIAS
    # split-K partials: AUTO's split plan on the pack's tiled width (128
    # columns per 256-column packed tile), none for decode or full grids
    assert L.swiglu_gemm_workspace_bytes(1, 3584, 18944) == 0
    assert L.swiglu_gemm_workspace_bytes(4096, 8192, 29568) == 0
    need = L.swiglu_gemm_workspace_bytes(128, 18944, 3584)
    nt = 14 * 128
    assert need > 0 and need % (128 * 2 * nt * 4) == 0 and need // (128 * 2 * nt * 4) >= 2
    assert L.swiglu_gemm_workspace_bytes(128, 18940, 3584) == 0     # K not a multiple of 8
    # a workspace that holds the partials is checked like the fused product's
    assert G(A_, WP_, Y_, 128, 18944, 3584, WS_ + 8, need, None) == MISAL
    assert G(A_, WP_, Y_, 128, 18944, 3584, Y_ + 4096, need, None) == ALIAS
    assert G(A_, WP_, Y_, 128, 18944, 3584, WP_ + 4096, need, None) == ALIAS
    # the MLP's workspace covers both steps
    M_, K_, N_ = 128, 3584, 18944
    assert L.swiglu_mlp_workspace_bytes(M_, K_, N_, 0) == max(L.swiglu_workspace_bytes(M_, K_, N_, 0),
                                                               L.swiglu_gemm_workspace_bytes(M_, N_, K_)) > 0
    assert L.swiglu_mlp_workspace_bytes(M_, K_, N_, 9) == 0
    P = L.swiglu_gemm_pack_weight
    assert P(W1_, W1_ + 16, 64, 64, None) == ALIAS
    assert P(W1_, WP_, 64, 63, None) == UNSUP
    assert P(None, WP_, 64, 64, None) == NULLP
    U = L.swiglu_unfused_packed
    assert U(None, None, None, None, None, None, 0, 64, 64, None) == OK
    assert U(A_, W1_, W2_, Y_, Y_, WS_, 4, 64, 64, None) == ALIAS
    assert U(A_, W1_, W2_, W1_ + 64, WP_, WS_, 4, 64, 64, None) == ALIAS
    assert U(A_, W1_, W2_, None, WP_, WS_, 4, 64, 64, None) == NULLP


def test_interleaved_errors():
    L = sw.lib()
    assert L.swiglu_pack_weights_interleaved(W1_, W2_, W1_ + 16, 64, 64, None) == ALIAS
    assert L.swiglu_pack_weights_interleaved(W1_, W2_, WP_, 63, 64, None) == UNSUP
    assert L.swiglu_pack_weights_interleaved(W1_, None, WP_, 64, 64, None) == NULLP
    assert L.swiglu_unpack_weights_interleaved(WP_, W1_, W1_, 64, 64, None) == ALIAS
    assert L.swiglu_unpack_weights_interleaved(WP_ + 4, W1_, W2_, 64, 64, None) == MISAL
    F = L.swiglu_fused_packed_interleaved
    assert F(None, None, None, 0, 64, 64, None) == OK
    assert F(A_, WP_, Y_, 4, 64, 60, None) == UNSUP
    assert F(A_, None, Y_, 4, 64, 64, None) == NULLP
    assert F(A_, WP_, Y_ + 2, 4, 64, 64, None) == MISAL
    assert F(A_, WP_, WP_ + 64, 4, 64, 64, None) == ALIAS
    assert F(A_, WP_, A_ + 16, 4, 64, 64, None) == ALIAS


def test_fp8_errors():
    L = sw.lib()
    # one 32 KiB block per 128 columns and 128 k
    assert L.swiglu_packed_bytes_fp8(896, 4864) == 38 * 7 * 32768
    assert L.swiglu_packed_bytes_fp8(8, 64) == 0          # K not a multiple of 16
    assert L.swiglu_packed_bytes_fp8(144, 136) == 2 * 2 * 32768
    F = L.swiglu_fused_packed_fp8
    assert F(None, None, None, 0, 64, 64, 1.0, 1.0, None) == OK
    assert F(A_, WP_, Y_, 4, 72, 64, 1.0, 1.0, None) == UNSUP
    assert F(A_, None, Y_, 4, 64, 64, 1.0, 1.0, None) == NULLP
    assert F(A_ + 8, WP_, Y_, 4, 64, 64, 1.0, 1.0, None) == MISAL
    assert F(A_, WP_, A_ + 128, 4, 64, 64, 1.0, 1.0, None) == ALIAS
    P = L.swiglu_pack_weights_fp8
    assert P(W1_, W2_, WP_, 72, 64, None) == UNSUP
    assert P(W1_, None, WP_, 64, 64, None) == NULLP
    assert P(W1_, W2_, W1_ + 16, 64, 64, None) == ALIAS


def test_noalloc_host_checks():
    """The no-allocation entry point validates like swiglu_fused_packed and
    rejects, before any HIP call, a schedule whose split-K partial sums do not
    fit the library's scratch array."""
    L = sw.lib()
    F = L.swiglu_fused_packed_noalloc
    assert F(None, None, None, 0, 64, 64, 0, None) == OK
    assert F(A_, WP_, Y_, 4, 60, 64, 0, None) == UNSUP
    assert F(A_, WP_, Y_, 4, 64, 64, 9, None) == VARIANT
    assert F(A_, WP_, Y_, 65, 64, 64, 3, None) == VARIANT
    assert F(A_, None, Y_, 4, 64, 64, 0, None) == NULLP
    big = L.swiglu_workspace_bytes(128, 3584, 18944, 2)
    assert big > sw.NOALLOC_SCRATCH_BYTES
    assert F(A_, WP_, Y_, 128, 3584, 18944, 2, None) == WS


def test_workspace_holds_fp32_partials():
    L = sw.lib()
    # split-K workspace = splits x M x 2N fp32 partial sums; zero for the
    # data-parallel and decode schedules
    for M, K, N in [(1, 3584, 18944), (16, 3584, 18944), (128, 3584, 18944), (32, 8192, 29568)]:
        b = L.swiglu_workspace_bytes(M, K, N, 2)
        per_split = M * 2 * N * 4
        assert b > 0 and b % per_split == 0 and 2 <= b // per_split <= K // 128
        assert L.swiglu_workspace_bytes(M, K, N, 1) == 0
        assert L.swiglu_workspace_bytes(M, K, N, 3) == 0


def test_probe_argument_errors():
    L = sw.lib()
    assert L.swiglu_probe_mfma(None, 1, 1, None) == NULLP
    assert L.swiglu_probe_mfma(Y_, 0, 1, None) == SHAPE
    assert L.swiglu_probe_read(A_, 15, Y_, 1, None) == SHAPE
    assert L.swiglu_probe_read(A_ + 4, 64, Y_, 1, None) == MISAL


def test_binding_argument_errors():
    """The binding names what is wrong before any call into the library."""
    import torch
    a = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        sw._dev_bf16([1, 2], "A")
    with pytest.raises(ValueError, match="GPU tensor"):
        sw._dev_bf16(a, "A")
    with pytest.raises(ValueError, match="GPU tensor"):
        sw._dev_bf16(a.float(), "A")


def test_binding_rejects_wrong_sizes():
    """Buffers the library would read or write past their end are rejected by
    the binding before the call (the C ABI trusts the sizes it is given)."""
    import torch
    bf = torch.bfloat16
    M, K, N = 4, 64, 128
    A = torch.zeros(M, K, dtype=bf)
    W = torch.zeros(K, N, dtype=bf)
    need = sw.swiglu_packed_bytes(K, N)
    small_wp = torch.zeros(need // 2 - 8, dtype=bf)
    with pytest.raises(ValueError, match="Wp holds"):
        sw.swiglu_fused_packed(A, small_wp, N)
    with pytest.raises(ValueError, match="Wp holds"):
        sw.swiglu_fused_packed_interleaved(A, small_wp, N)
    with pytest.raises(ValueError, match="Wp holds"):
        sw.swiglu_unpack_weights(small_wp, K, N)
    wp = torch.zeros(need // 2, dtype=bf)
    with pytest.raises(ValueError, match="Y must be"):
        sw.swiglu_fused_packed(A, wp, N, Y=torch.zeros(M, N - 8, dtype=bf))
    with pytest.raises(ValueError, match="Y must be"):
        sw.swiglu_fused(A, W, W, Y=torch.zeros(M + 1, N, dtype=bf))
    with pytest.raises(ValueError, match="W must be"):
        sw.swiglu_gemm_bf16(A, torch.zeros(K + 8, N, dtype=bf))
    with pytest.raises(ValueError, match="C must be"):
        sw.swiglu_gemm_bf16(A, W, C=torch.zeros(M, N + 8, dtype=bf))
    with pytest.raises(ValueError, match="U must be"):
        sw.swiglu_unfused(A, W, W, U=torch.zeros(M, 8, dtype=bf))
    with pytest.raises(ValueError, match="Y must be"):
        sw.swiglu_silu_mul(torch.zeros(M, N, dtype=bf), torch.zeros(M, N, dtype=bf), Y=torch.zeros(M, 8, dtype=bf))
    wg = torch.zeros(sw.swiglu_gemm_packed_bytes(K, N) // 2, dtype=bf)
    w3g = torch.zeros(sw.swiglu_gemm_packed_bytes(N, K) // 2, dtype=bf)
    with pytest.raises(ValueError, match="W3g holds"):
        sw.swiglu_mlp_packed(A, wp, torch.zeros(K, N, dtype=bf), N)
    with pytest.raises(ValueError, match="Z must be"):
        sw.swiglu_mlp_down(torch.zeros(M, N, dtype=bf), w3g, K, Z=torch.zeros(M, 8, dtype=bf))
    with pytest.raises(ValueError, match="W3g holds"):
        sw.swiglu_mlp_down(torch.zeros(M, N, dtype=bf), w3g[:-8], K)
    with pytest.raises(ValueError, match="W3g holds"):
        sw.swiglu_mlp_unfused(A, wg, wg, torch.zeros(K, K, dtype=bf), N)
    with pytest.raises(ValueError, match="W2g holds"):
        sw.swiglu_mlp_unfused(A, wg, wg[:-8], w3g, N)
    with pytest.raises(ValueError, match="Wg holds"):
        sw.swiglu_gemm_packed(A, wg[:-8], N)
    with pytest.raises(ValueError, match="C must be"):
        sw.swiglu_gemm_packed(A, wg, N, C=torch.zeros(M, N - 8, dtype=bf))
    with pytest.raises(ValueError, match="W1g holds"):
        sw.swiglu_unfused_packed(A, wg[:-8], wg, N)
    with pytest.raises(ValueError, match="Wg holds"):
        sw.swiglu_gemm_pack_weight(W, Wg=wg[:-8])
    # the pack entry points read W2 at W1's shape; the interleaved unpack
    # reads a whole packed buffer
    with pytest.raises(ValueError, match="W2 must be"):
        sw.swiglu_pack_weights(W, torch.zeros(K - 8, N, dtype=bf))
    with pytest.raises(ValueError, match="W2 must be"):
        sw.swiglu_pack_weights_interleaved(W, torch.zeros(K, N - 8, dtype=bf))
    with pytest.raises(ValueError, match="W2 must be"):
        sw.swiglu_pack_weights_fp8(torch.zeros(K, N, dtype=torch.uint8), torch.zeros(K, 8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="Wp holds"):
        sw.swiglu_unpack_weights_interleaved(small_wp, K, N)
    need8 = int(sw.lib().swiglu_packed_bytes_fp8(K, N))
    with pytest.raises(ValueError, match="Wp holds"):
        sw.swiglu_fused_packed_fp8(torch.zeros(M, K, dtype=torch.uint8), torch.zeros(need8 - 16, dtype=torch.uint8),
                                   N, 1.0, 1.0)


def test_auto_dispatch_at_workload_shapes():
    """AUTO's choice is host logic (no device work): decode up to 32 rows and,
    up to 64 rows, while the 32-column weight panels number fewer than the CUs;
    the data-parallel streaming schedule otherwise.  Without a device the
    library plans for 256 CUs, the MI355X count, so these are the choices the
    GPU runs make."""
    L = sw.lib()
    DP, DEC = 1, 3
    cases = [
        (64, 896, 4864, DEC),        # tiny: 152 panels < 256 CUs
        (4096, 896, 4864, DP),       # 0.5B prefill
        (1, 3584, 18944, DEC), (16, 3584, 18944, DEC), (32, 3584, 18944, DEC),
        (64, 3584, 18944, DP),       # 592 panels >= 256 CUs: panel schedule
        (128, 3584, 18944, DP), (8192, 3584, 18944, DP),
        (32, 8192, 29568, DEC), (4096, 8192, 29568, DP),
        (48, 6144, 12288, DP),       # 384 panels >= 256 CUs
        (33, 64, 128, DEC),          # 4 panels
    ]
    for M, K, N, want in cases:
        assert L.swiglu_choose_variant(M, K, N) == want, (M, K, N)
    # no AUTO choice needs a workspace at these shapes
    for M, K, N, _ in cases:
        assert L.swiglu_workspace_bytes(M, K, N, 0) == 0, (M, K, N)


def test_auto_split_k_choice_and_workspace():
    """Split-K only while the data-parallel tiles fill under half the CUs, with
    at most K / (16 M) splits; its workspace is S fp32 partial sums of Gate and
    Up, S * M * 2N * 4 bytes."""
    L = sw.lib()
    cases = [
        # M, K, N, splits: 8 tiles of 128x128 -> cap K/(16M) = 4
        (128, 8192, 1024, 4),
        # 16 tiles -> cap 2
        (256, 8192, 1024, 2),
        # 4 tiles -> cap 4096 // 1600 = 2
        (100, 4096, 512, 2),
    ]
    for M, K, N, S in cases:
        assert L.swiglu_choose_variant(M, K, N) == 2, (M, K, N)
        assert L.swiglu_workspace_bytes(M, K, N, 0) == S * M * 2 * N * 4, (M, K, N)
    # K too short for two splits of at least 16 M: data-parallel, no workspace
    assert L.swiglu_choose_variant(128, 1024, 1024) == 1
    assert L.swiglu_workspace_bytes(128, 1024, 1024, 0) == 0
    # enough data-parallel tiles to fill half the CUs: data-parallel
    assert L.swiglu_choose_variant(2048, 8192, 256) == 1
