"""Python binding of libswiglu (the fused SwiGLU gated-MLP product on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libswiglu.so``; this module checks tensor types, allocates
outputs with torch (device memory) and passes raw pointers plus the current
torch stream through the C ABI declared in ``include/swiglu.h``.  The function
names are the C entry points' names.  There is no fallback: if the library is
missing or the device is not a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import inputs  # noqa: F401  (seeded input generators)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswiglu.so")

SWIGLU_OK = 0
SWIGLU_ERR_HIP = 8
VARIANT_AUTO = 0
VARIANT_DATA_PARALLEL = 1
VARIANT_SPLIT_K = 2
VARIANT_DECODE = 3
VARIANT_SEQUENTIAL = 4
VARIANTS = {"auto": VARIANT_AUTO, "data_parallel": VARIANT_DATA_PARALLEL, "split_k": VARIANT_SPLIT_K,
            "decode": VARIANT_DECODE, "sequential": VARIANT_SEQUENTIAL}

# Every entry point of include/swiglu.h with its ctypes signature.
_I64 = ctypes.c_int64
_P = ctypes.c_void_p
SIGNATURES = {
    "swiglu_abi_version": ([], ctypes.c_int),
    "swiglu_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "swiglu_last_hip_error": ([], ctypes.c_int),
    "swiglu_device_cu_count": ([], ctypes.c_int),
    "swiglu_fused": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "swiglu_packed_bytes": ([_I64, _I64], ctypes.c_size_t),
    "swiglu_pack_weights": ([_P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "swiglu_unpack_weights": ([_P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "swiglu_workspace_bytes": ([_I64, _I64, _I64, ctypes.c_int], ctypes.c_size_t),
    "swiglu_fused_packed": ([_P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, ctypes.c_int, _P],
                            ctypes.c_int),
    "swiglu_choose_variant": ([_I64, _I64, _I64], ctypes.c_int),
    "swiglu_fused_packed_noalloc": ([_P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P], ctypes.c_int),
    "swiglu_packed_bytes_fp8": ([_I64, _I64], ctypes.c_size_t),
    "swiglu_pack_weights_fp8": ([_P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "swiglu_fused_packed_fp8": ([_P, _P, _P, _I64, _I64, _I64, ctypes.c_float, ctypes.c_float, _P], ctypes.c_int),
    "swiglu_pack_weights_interleaved": ([_P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "swiglu_unpack_weights_interleaved": ([_P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "swiglu_fused_packed_interleaved": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "swiglu_gemm_bf16": ([_P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "swiglu_gemm_packed_bytes": ([_I64, _I64], ctypes.c_size_t),
    "swiglu_gemm_pack_weight": ([_P, _P, _I64, _I64, _P], ctypes.c_int),
    "swiglu_gemm_workspace_bytes": ([_I64, _I64, _I64], ctypes.c_size_t),
    "swiglu_gemm_packed": ([_P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "swiglu_unfused_packed": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "swiglu_silu_mul": ([_P, _P, _P, _I64, _P], ctypes.c_int),
    "swiglu_unfused": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "swiglu_mlp_packed": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, ctypes.c_int, _P],
                          ctypes.c_int),
    "swiglu_mlp_workspace_bytes": ([_I64, _I64, _I64, ctypes.c_int], ctypes.c_size_t),
    "swiglu_mlp_unfused": ([_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P],
                           ctypes.c_int),
    "swiglu_mlp_down": ([_P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P], ctypes.c_int),
    # include/swiglu_probe.h (diagnostic ceilings)
    "swiglu_probe_mfma": ([_P, ctypes.c_int, ctypes.c_int, _P], ctypes.c_int),
    "swiglu_probe_read": ([_P, ctypes.c_size_t, _P, ctypes.c_int, _P], ctypes.c_int),
}

_lock = threading.Lock()
_lib = None


class SwigluError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        msg = "%s failed: %s (status %d)" % (fn, status_str(status), status)
        if status == SWIGLU_ERR_HIP:
            msg += ", hipError_t %d" % hip_error
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


def lib():
    """The loaded libswiglu (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libswiglu.so is not built (%s); run "
                                   "`python -m swiglu_gated_mlp_amd.build`" % LIB_PATH)
            handle = ctypes.CDLL(LIB_PATH)
            for name, (argt, rest) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.argtypes = argt
                fn.restype = rest
            _lib = handle
        return _lib


def status_str(status: int) -> str:
    return lib().swiglu_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != SWIGLU_OK:
        raise SwigluError(fn, status, lib().swiglu_last_hip_error() if status == SWIGLU_ERR_HIP else 0)


def _dev_bf16(t: torch.Tensor, name: str) -> int:
    # fast path first (a call's host time matters for small shapes); the
    # checks below only name what is wrong
    if isinstance(t, torch.Tensor) and t.is_cuda and t.dtype is torch.bfloat16 and t.is_contiguous():
        return t.data_ptr()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16 (got %s)" % (name, t.dtype))
    raise ValueError("%s must be contiguous" % name)


def _shape(t, shape, name: str) -> None:
    """A tensor the library reads or writes must hold exactly this shape (the C
    ABI takes bare pointers and trusts the sizes)."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be %s (got %s)" % (name, list(shape), list(t.shape)))


_packed_need: dict = {}


def _packed_at_least(Wp, K: int, N: int, name: str = "Wp", fp8: bool = False) -> None:
    """Wp must hold at least the packed weights of a [K,N] pair."""
    key = (K, N, fp8)
    need = _packed_need.get(key)
    if need is None:
        need = int(lib().swiglu_packed_bytes_fp8(K, N) if fp8 else lib().swiglu_packed_bytes(K, N))
        _packed_need[key] = need
    if need == 0:
        raise ValueError("invalid weight shape [%d,%d]" % (K, N))
    if Wp.numel() * Wp.element_size() < need:
        raise ValueError("%s holds %d bytes; packed [%d,%d] weights need %d"
                         % (name, Wp.numel() * Wp.element_size(), K, N, need))


_gemm_need: dict = {}


def _gemm_packed_at_least(Wg, K: int, N: int, name: str = "Wg") -> None:
    """Wg must hold at least the single-weight pack of a [K,N] weight."""
    need = _gemm_need.get((K, N))
    if need is None:
        need = _gemm_need[(K, N)] = int(lib().swiglu_gemm_packed_bytes(K, N))
    if need == 0:
        raise ValueError("invalid weight shape [%d,%d]" % (K, N))
    if Wg.numel() * Wg.element_size() < need:
        raise ValueError("%s holds %d bytes; a packed [%d,%d] weight needs %d"
                         % (name, Wg.numel() * Wg.element_size(), K, N, need))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def swiglu_abi_version() -> int:
    return int(lib().swiglu_abi_version())


def swiglu_device_cu_count() -> int:
    return int(lib().swiglu_device_cu_count())


def swiglu_fused(A: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor, Y: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Y = SiLU(A @ W1) * (A @ W2) from row-major weights; returns Y [M,N] bf16."""
    M, K = A.shape
    N = W1.shape[1]
    if W1.shape != (K, N) or W2.shape != (K, N):
        raise ValueError("W1, W2 must be [K,N] = [%d,%d]" % (K, N))
    _shape(Y, (M, N), "Y")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    st = lib().swiglu_fused(_dev_bf16(A, "A"), _dev_bf16(W1, "W1"), _dev_bf16(W2, "W2"),
                            _dev_bf16(Y, "Y"), M, K, N, _stream(stream))
    _check("swiglu_fused", st)
    return Y


def swiglu_packed_bytes(K: int, N: int) -> int:
    return int(lib().swiglu_packed_bytes(K, N))


def swiglu_pack_weights(W1: torch.Tensor, W2: torch.Tensor, Wp: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Pack W1, W2 [K,N] into the per-128-column-tile [W1 | W2] layout."""
    K, N = W1.shape
    _shape(W2, (K, N), "W2")
    nbytes = swiglu_packed_bytes(K, N)
    if nbytes == 0:
        raise ValueError("invalid weight shape [%d,%d]" % (K, N))
    if Wp is None:
        Wp = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=W1.device)
    elif Wp.numel() * Wp.element_size() < nbytes:
        raise ValueError("Wp too small: need %d bytes" % nbytes)
    st = lib().swiglu_pack_weights(_dev_bf16(W1, "W1"), _dev_bf16(W2, "W2"), _dev_bf16(Wp, "Wp"),
                                   K, N, _stream(stream))
    _check("swiglu_pack_weights", st)
    return Wp


def swiglu_unpack_weights(Wp: torch.Tensor, K: int, N: int, stream=None):
    """Inverse of swiglu_pack_weights; returns (W1, W2)."""
    _packed_at_least(Wp, K, N)
    W1 = torch.empty((K, N), dtype=torch.bfloat16, device=Wp.device)
    W2 = torch.empty((K, N), dtype=torch.bfloat16, device=Wp.device)
    st = lib().swiglu_unpack_weights(_dev_bf16(Wp, "Wp"), _dev_bf16(W1, "W1"), _dev_bf16(W2, "W2"),
                                     K, N, _stream(stream))
    _check("swiglu_unpack_weights", st)
    return W1, W2


def _dev_u8(t: torch.Tensor, name: str) -> int:
    if isinstance(t, torch.Tensor) and t.is_cuda and t.dtype is torch.uint8 and t.is_contiguous():
        return t.data_ptr()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if t.dtype != torch.uint8:
        raise TypeError("%s must be uint8 FP8 E4M3 bytes (got %s)" % (name, t.dtype))
    raise ValueError("%s must be contiguous" % name)


def swiglu_pack_weights_fp8(W1: torch.Tensor, W2: torch.Tensor, stream=None) -> torch.Tensor:
    """Pack FP8 E4M3 weight bytes W1, W2 [K,N] (uint8) for swiglu_fused_packed_fp8."""
    K, N = W1.shape
    _shape(W2, (K, N), "W2")
    _dev_u8(W1, "W1")
    _dev_u8(W2, "W2")
    nbytes = int(lib().swiglu_packed_bytes_fp8(K, N))
    if nbytes == 0:
        raise ValueError("invalid FP8 weight shape [%d,%d] (K must be a multiple of 16)" % (K, N))
    Wp = torch.empty(nbytes, dtype=torch.uint8, device=W1.device)
    st = lib().swiglu_pack_weights_fp8(_dev_u8(W1, "W1"), _dev_u8(W2, "W2"), _dev_u8(Wp, "Wp"), K, N,
                                       _stream(stream))
    _check("swiglu_pack_weights_fp8", st)
    return Wp


def swiglu_fused_packed_fp8(A8: torch.Tensor, Wp: torch.Tensor, N: int, sg: float, su: float,
                            Y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = bf16(SiLU(sg * A8 W1_8) * (su * A8 W2_8)) from FP8 E4M3 bytes."""
    M, K = A8.shape
    _packed_at_least(Wp, K, N, fp8=True)
    _shape(Y, (M, N), "Y")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=A8.device) if Y is None else Y
    st = lib().swiglu_fused_packed_fp8(_dev_u8(A8, "A8"), _dev_u8(Wp, "Wp"), _dev_bf16(Y, "Y"), M, K, N,
                                       float(sg), float(su), _stream(stream))
    _check("swiglu_fused_packed_fp8", st)
    return Y


def swiglu_pack_weights_interleaved(W1: torch.Tensor, W2: torch.Tensor, Wp: torch.Tensor | None = None,
                                    stream=None) -> torch.Tensor:
    """Pack W1, W2 [K,N] column-granular interleaved (Gate even, Up odd rows)."""
    K, N = W1.shape
    _shape(W2, (K, N), "W2")
    nbytes = swiglu_packed_bytes(K, N)
    if nbytes == 0:
        raise ValueError("invalid weight shape [%d,%d]" % (K, N))
    if Wp is None:
        Wp = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=W1.device)
    elif Wp.numel() * Wp.element_size() < nbytes:
        raise ValueError("Wp too small: need %d bytes" % nbytes)
    st = lib().swiglu_pack_weights_interleaved(_dev_bf16(W1, "W1"), _dev_bf16(W2, "W2"), _dev_bf16(Wp, "Wp"),
                                               K, N, _stream(stream))
    _check("swiglu_pack_weights_interleaved", st)
    return Wp


def swiglu_unpack_weights_interleaved(Wp: torch.Tensor, K: int, N: int, stream=None):
    """Inverse of swiglu_pack_weights_interleaved; returns (W1, W2)."""
    _packed_at_least(Wp, K, N)
    W1 = torch.empty((K, N), dtype=torch.bfloat16, device=Wp.device)
    W2 = torch.empty((K, N), dtype=torch.bfloat16, device=Wp.device)
    st = lib().swiglu_unpack_weights_interleaved(_dev_bf16(Wp, "Wp"), _dev_bf16(W1, "W1"),
                                                 _dev_bf16(W2, "W2"), K, N, _stream(stream))
    _check("swiglu_unpack_weights_interleaved", st)
    return W1, W2


def swiglu_fused_packed_interleaved(A: torch.Tensor, Wp: torch.Tensor, N: int, Y: torch.Tensor | None = None,
                                    stream=None) -> torch.Tensor:
    """Y = SiLU(A W1) * (A W2) from column-interleaved packed weights."""
    M, K = A.shape
    _packed_at_least(Wp, K, N)
    _shape(Y, (M, N), "Y")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=A.device) if Y is None else Y
    st = lib().swiglu_fused_packed_interleaved(_dev_bf16(A, "A"), _dev_bf16(Wp, "Wp"), _dev_bf16(Y, "Y"),
                                               M, K, N, _stream(stream))
    _check("swiglu_fused_packed_interleaved", st)
    return Y


def swiglu_workspace_bytes(M: int, K: int, N: int, variant: int = VARIANT_AUTO) -> int:
    return int(lib().swiglu_workspace_bytes(M, K, N, int(variant)))


_ws_need: dict = {}


def _cached_need(kind: str, args: tuple, device: torch.device) -> int:
    """swiglu_gemm_workspace_bytes ("gemm") or swiglu_mlp_workspace_bytes
    ("mlp") of args, remembered per device (the plans depend only on the
    shape and the device's CU count)."""
    key = (kind, args, device.index)
    need = _ws_need.get(key)
    if need is None:
        fn = swiglu_gemm_workspace_bytes if kind == "gemm" else swiglu_mlp_workspace_bytes
        need = _ws_need[key] = fn(*args)
    return need


def _workspace_need(M: int, K: int, N: int, variant: int, device: torch.device) -> int:
    """swiglu_workspace_bytes, remembered per (shape, variant, device): the
    plan depends only on these and the device's CU count."""
    key = (M, K, N, variant, device.index)
    need = _ws_need.get(key)
    if need is None:
        need = _ws_need[key] = swiglu_workspace_bytes(M, K, N, variant)
    return need


def swiglu_gemm_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().swiglu_gemm_workspace_bytes(M, K, N))


def swiglu_mlp_workspace_bytes(M: int, K: int, N: int, variant: int = VARIANT_AUTO) -> int:
    return int(lib().swiglu_mlp_workspace_bytes(M, K, N, int(variant)))


def _resolve_workspace(workspace, need: int, device: torch.device, s: int):
    """(pointer-able tensor or None, its bytes) for a call needing `need`
    bytes: a caller tensor as given, a Workspace grown to `need`, or the
    cached per-stream Workspace."""
    if need == 0 and not isinstance(workspace, torch.Tensor):
        ws = None
    elif isinstance(workspace, Workspace):
        ws = workspace.get(need, s)
    elif workspace is None:
        ws = _workspace_for(device, s).get(need, s)
    else:
        ws = workspace
    if ws is not None and ws.device.type != "cuda":
        raise ValueError("workspace must be a GPU tensor")
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def swiglu_choose_variant(M: int, K: int, N: int) -> int:
    return int(lib().swiglu_choose_variant(M, K, N))


class Workspace:
    """Device scratch for the split-K schedule (fp32 partial sums), grown on
    demand.  Its contents never need clearing.  One Workspace must not be
    shared by calls that may run concurrently."""

    def __init__(self, device=None):
        self.device = torch.device(device or "cuda")
        self.buf: torch.Tensor | None = None

    def get(self, nbytes: int, stream: int | None = None) -> torch.Tensor | None:
        """A buffer of at least nbytes.  A larger buffer replaces a smaller
        one; it is allocated on `stream` (a raw handle: the stream of the
        calls that will use it), so the caching allocator hands the old
        buffer's memory out again only to work ordered after those calls."""
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = None
            if stream is None or stream == torch.cuda.current_stream(self.device).cuda_stream:
                self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            else:
                with torch.cuda.stream(torch.cuda.ExternalStream(stream, device=self.device)):
                    self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws: dict = {}


def _workspace_for(device: torch.device, stream_handle: int) -> Workspace:
    key = (device.index, stream_handle)
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(device)
    return ws


def swiglu_fused_packed(A: torch.Tensor, Wp: torch.Tensor, N: int, Y: torch.Tensor | None = None,
                        workspace: torch.Tensor | Workspace | None = None, variant: int = VARIANT_AUTO,
                        stream=None) -> torch.Tensor:
    """Y = SiLU(A W1) * (A W2) from packed weights; returns Y [M,N] bf16.

    ``workspace`` may be a uint8 tensor of at least swiglu_workspace_bytes()
    bytes, a Workspace, or None (a cached per-stream Workspace is used)."""
    M, K = A.shape
    _packed_at_least(Wp, K, N)
    _shape(Y, (M, N), "Y")
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    s = _stream(stream)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    ws, ws_bytes = _resolve_workspace(workspace, _workspace_need(M, K, N, int(variant), A.device), A.device, s)
    st = lib().swiglu_fused_packed(_dev_bf16(A, "A"), _dev_bf16(Wp, "Wp"), _dev_bf16(Y, "Y"), M, K, N,
                                   _ptr(ws), ws_bytes, int(variant), s)
    _check("swiglu_fused_packed", st)
    return Y


#: bytes of the library's per-device scratch array (swiglu_fused_packed_noalloc)
NOALLOC_SCRATCH_BYTES = 32 << 20


def swiglu_fused_packed_noalloc(A: torch.Tensor, Wp: torch.Tensor, Y: torch.Tensor, variant: int = VARIANT_AUTO,
                                stream=None) -> torch.Tensor:
    """swiglu_fused_packed into the caller's Y with no allocation: split-K
    partial sums go to the library's own device scratch array (the binding
    allocates nothing either; Y [M,N] is required)."""
    M, K = A.shape
    N = Y.shape[1]
    _packed_at_least(Wp, K, N)
    _shape(Y, (M, N), "Y")
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    st = lib().swiglu_fused_packed_noalloc(_dev_bf16(A, "A"), _dev_bf16(Wp, "Wp"), _dev_bf16(Y, "Y"), M, K, N,
                                           int(variant), _stream(stream))
    _check("swiglu_fused_packed_noalloc", st)
    return Y


def swiglu_gemm_bf16(A: torch.Tensor, W: torch.Tensor, C: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """C = bf16(A @ W) with fp32 accumulation (one GEMM of the unfused pipeline)."""
    M, K = A.shape
    N = W.shape[1]
    _shape(W, (K, N), "W")
    _shape(C, (M, N), "C")
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    st = lib().swiglu_gemm_bf16(_dev_bf16(A, "A"), _dev_bf16(W, "W"), _dev_bf16(C, "C"), M, K, N,
                                _stream(stream))
    _check("swiglu_gemm_bf16", st)
    return C


def swiglu_gemm_packed_bytes(K: int, N: int) -> int:
    return int(lib().swiglu_gemm_packed_bytes(K, N))


def swiglu_gemm_pack_weight(W: torch.Tensor, Wg: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Pack one weight W [K,N] for swiglu_gemm_packed (256 columns per packed
    tile, the fused pack's block layout)."""
    K, N = W.shape
    nbytes = swiglu_gemm_packed_bytes(K, N)
    if nbytes == 0:
        raise ValueError("invalid weight shape [%d,%d]" % (K, N))
    if Wg is None:
        Wg = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=W.device)
    else:
        _gemm_packed_at_least(Wg, K, N)
    st = lib().swiglu_gemm_pack_weight(_dev_bf16(W, "W"), _dev_bf16(Wg, "Wg"), K, N, _stream(stream))
    _check("swiglu_gemm_pack_weight", st)
    return Wg


def swiglu_gemm_packed(A: torch.Tensor, Wg: torch.Tensor, N: int, C: torch.Tensor | None = None,
                       workspace: torch.Tensor | Workspace | None = None, stream=None) -> torch.Tensor:
    """C = bf16(A @ W) with fp32 accumulation from a single-weight pack.
    ``workspace`` as in swiglu_fused_packed (None: the cached per-stream one,
    so split-K runs where the plan asks for it)."""
    M, K = A.shape
    _gemm_packed_at_least(Wg, K, N)
    _shape(C, (M, N), "C")
    C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device) if C is None else C
    s = _stream(stream)
    ws, ws_bytes = _resolve_workspace(workspace, _cached_need("gemm", (M, K, N), A.device), A.device, s)
    st = lib().swiglu_gemm_packed(_dev_bf16(A, "A"), _dev_bf16(Wg, "Wg"), _dev_bf16(C, "C"), M, K, N,
                                  _ptr(ws), ws_bytes, s)
    _check("swiglu_gemm_packed", st)
    return C


def swiglu_unfused_packed(A: torch.Tensor, W1g: torch.Tensor, W2g: torch.Tensor, N: int,
                          G: torch.Tensor | None = None, U: torch.Tensor | None = None,
                          Y: torch.Tensor | None = None, stream=None):
    """The unfused pipeline on single-weight packs: G = A@W1, U = A@W2 (bf16,
    in memory), Y = SiLU(G)*U.  Returns (G, U, Y)."""
    M, K = A.shape
    _gemm_packed_at_least(W1g, K, N, "W1g")
    _gemm_packed_at_least(W2g, K, N, "W2g")
    for t, name in ((G, "G"), (U, "U"), (Y, "Y")):
        _shape(t, (M, N), name)
    mk = lambda: torch.empty((M, N), dtype=torch.bfloat16, device=A.device)  # noqa: E731
    G = mk() if G is None else G
    U = mk() if U is None else U
    Y = mk() if Y is None else Y
    st = lib().swiglu_unfused_packed(_dev_bf16(A, "A"), _dev_bf16(W1g, "W1g"), _dev_bf16(W2g, "W2g"),
                                     _dev_bf16(G, "G"), _dev_bf16(U, "U"), _dev_bf16(Y, "Y"), M, K, N,
                                     _stream(stream))
    _check("swiglu_unfused_packed", st)
    return G, U, Y


def swiglu_silu_mul(G: torch.Tensor, U: torch.Tensor, Y: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Y = bf16(SiLU(G) * U), element-wise (the unfused pipeline's activation)."""
    if G.shape != U.shape:
        raise ValueError("G and U shapes differ")
    _shape(Y, G.shape, "Y")
    if Y is None:
        Y = torch.empty_like(G)
    st = lib().swiglu_silu_mul(_dev_bf16(G, "G"), _dev_bf16(U, "U"), _dev_bf16(Y, "Y"), G.numel(),
                               _stream(stream))
    _check("swiglu_silu_mul", st)
    return Y


def swiglu_unfused(A: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor, G: torch.Tensor | None = None,
                   U: torch.Tensor | None = None, Y: torch.Tensor | None = None, stream=None):
    """The unfused pipeline: G = A@W1, U = A@W2 (bf16, in memory), Y = SiLU(G)*U.
    Returns (G, U, Y)."""
    M, K = A.shape
    N = W1.shape[1]
    for t, shape, name in ((W1, (K, N), "W1"), (W2, (K, N), "W2"), (G, (M, N), "G"), (U, (M, N), "U"),
                           (Y, (M, N), "Y")):
        _shape(t, shape, name)
    mk = lambda: torch.empty((M, N), dtype=torch.bfloat16, device=A.device)  # noqa: E731
    G = mk() if G is None else G
    U = mk() if U is None else U
    Y = mk() if Y is None else Y
    st = lib().swiglu_unfused(_dev_bf16(A, "A"), _dev_bf16(W1, "W1"), _dev_bf16(W2, "W2"),
                              _dev_bf16(G, "G"), _dev_bf16(U, "U"), _dev_bf16(Y, "Y"), M, K, N,
                              _stream(stream))
    _check("swiglu_unfused", st)
    return G, U, Y


def swiglu_mlp_packed(A: torch.Tensor, Wp: torch.Tensor, W3g: torch.Tensor, N: int,
                      Y: torch.Tensor | None = None, Z: torch.Tensor | None = None,
                      workspace: torch.Tensor | Workspace | None = None, variant: int = VARIANT_AUTO,
                      stream=None):
    """The gated MLP block on packed weights: Y = SiLU(A W1) * (A W2), then
    Z = Y @ W3 (W3 [N,K] in the single-weight pack of swiglu_gemm_pack_weight,
    the down projection).  Returns (Y, Z)."""
    M, K = A.shape
    _packed_at_least(Wp, K, N)
    _gemm_packed_at_least(W3g, N, K, "W3g")
    for t, shape, name in ((Y, (M, N), "Y"), (Z, (M, K), "Z")):
        _shape(t, shape, name)
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    s = _stream(stream)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=A.device) if Y is None else Y
    Z = torch.empty((M, K), dtype=torch.bfloat16, device=A.device) if Z is None else Z
    ws, ws_bytes = _resolve_workspace(workspace, _cached_need("mlp", (M, K, N, int(variant)), A.device),
                                      A.device, s)
    st = lib().swiglu_mlp_packed(_dev_bf16(A, "A"), _dev_bf16(Wp, "Wp"), _dev_bf16(W3g, "W3g"),
                                 _dev_bf16(Y, "Y"), _dev_bf16(Z, "Z"), M, K, N, _ptr(ws), ws_bytes,
                                 int(variant), s)
    _check("swiglu_mlp_packed", st)
    return Y, Z


def swiglu_mlp_down(Y: torch.Tensor, W3g: torch.Tensor, K: int, Z: torch.Tensor | None = None,
                    workspace: torch.Tensor | Workspace | None = None, stream=None) -> torch.Tensor:
    """The MLP block's down projection alone: Z[M,K] = Y[M,N] @ W3[N,K], W3 in
    the single-weight pack; ``workspace`` as in swiglu_gemm_packed."""
    M, N = Y.shape
    _gemm_packed_at_least(W3g, N, K, "W3g")
    _shape(Z, (M, K), "Z")
    Z = torch.empty((M, K), dtype=torch.bfloat16, device=Y.device) if Z is None else Z
    s = _stream(stream)
    ws, ws_bytes = _resolve_workspace(workspace, _cached_need("gemm", (M, N, K), Y.device), Y.device, s)
    st = lib().swiglu_mlp_down(_dev_bf16(Y, "Y"), _dev_bf16(W3g, "W3g"), _dev_bf16(Z, "Z"), M, K, N,
                               _ptr(ws), ws_bytes, s)
    _check("swiglu_mlp_down", st)
    return Z


def swiglu_mlp_unfused(A: torch.Tensor, W1g: torch.Tensor, W2g: torch.Tensor, W3g: torch.Tensor, N: int,
                       G: torch.Tensor | None = None, U: torch.Tensor | None = None,
                       Y: torch.Tensor | None = None, Z: torch.Tensor | None = None,
                       workspace: torch.Tensor | Workspace | None = None, stream=None):
    """The gated MLP block, unfused, on single-weight packs: G, U through
    memory, Y = SiLU(G)*U, then Z = Y @ W3 (``workspace`` as in
    swiglu_gemm_packed, for the down projection).  Returns (Y, Z)."""
    M, K = A.shape
    _gemm_packed_at_least(W1g, K, N, "W1g")
    _gemm_packed_at_least(W2g, K, N, "W2g")
    _gemm_packed_at_least(W3g, N, K, "W3g")
    for t, shape, name in ((G, (M, N), "G"), (U, (M, N), "U"), (Y, (M, N), "Y"), (Z, (M, K), "Z")):
        _shape(t, shape, name)
    mk = lambda r, c: torch.empty((r, c), dtype=torch.bfloat16, device=A.device)  # noqa: E731
    G = mk(M, N) if G is None else G
    U = mk(M, N) if U is None else U
    Y = mk(M, N) if Y is None else Y
    Z = mk(M, K) if Z is None else Z
    s = _stream(stream)
    ws, ws_bytes = _resolve_workspace(workspace, _cached_need("gemm", (M, N, K), A.device), A.device, s)
    st = lib().swiglu_mlp_unfused(_dev_bf16(A, "A"), _dev_bf16(W1g, "W1g"), _dev_bf16(W2g, "W2g"),
                                  _dev_bf16(W3g, "W3g"), _dev_bf16(G, "G"), _dev_bf16(U, "U"),
                                  _dev_bf16(Y, "Y"), _dev_bf16(Z, "Z"), M, K, N, _ptr(ws), ws_bytes, s)
    _check("swiglu_mlp_unfused", st)
    return Y, Z


# ---------------------------------------------------------------------------
# diagnostic ceilings (include/swiglu_probe.h)
# ---------------------------------------------------------------------------

def swiglu_probe_mfma(sink: torch.Tensor, blocks: int, iters: int, stream=None) -> None:
    """MFMA-only loop: blocks x 4 waves x iters x 8 v_mfma_f32_32x32x16_bf16."""
    if sink.dtype != torch.float32 or sink.numel() < blocks * 256 or sink.device.type != "cuda":
        raise ValueError("sink must be a GPU float32 tensor of >= blocks*256 elements")
    _check("swiglu_probe_mfma", lib().swiglu_probe_mfma(sink.data_ptr(), blocks, iters, _stream(stream)))


def swiglu_probe_read(src: torch.Tensor, sink: torch.Tensor, blocks: int, stream=None) -> None:
    """Stream every byte of ``src`` through 16-byte loads."""
    nbytes = src.numel() * src.element_size()
    if src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if sink.dtype != torch.int32 or sink.numel() < blocks * 256 or sink.device.type != "cuda":
        raise ValueError("sink must be a GPU int32 tensor of >= blocks*256 elements")
    _check("swiglu_probe_read", lib().swiglu_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks,
                                                        _stream(stream)))
