"""CPU oracle for the fused SwiGLU product -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library neither links nor calls
it, and the two share no code: the only thing both sides see is the seeded
input generator in ``swiglu_gated_mlp_amd.inputs``, which holds none of the
method's arithmetic.

The arithmetic lives in ``oracle.c`` (plain C, fp32 accumulation in increasing
k, libm ``expf``, bit-exact round-to-nearest-even to bf16).  This module only
builds that file with gcc, loads it with ctypes and marshals numpy arrays.

Every function follows "Tile-Level Activation Overlap for Efficient LLM
Inference" as summarised on gist.science ("Summary"):

* ``swiglu``      -- Y = SiLU(A x W1) (.) (A x W2); Summary, "Problem Statement".
* ``unfused``     -- the two-GEMM + separate-activation pipeline whose Gate and
  Up go through memory; Summary, "Problem Statement" and "Results" (baseline).
* ``silu``        -- SiLU(x) = x / (1 + e^-x), the Swish applied to Gate;
  Summary, "Methodology", Kernel-1.
* ``bf16_rne``    -- rounding of the fp32 result to the bf16 output type.
* ``swiglu_fp8``  -- the product from FP8 E4M3 operands with per-tensor
  scales (the pages' remark that quantised GEMMs raise SwiGLU's relative cost,
  Summary, "Problem Statement"; the pages fix no scale convention, so per-tensor
  scales are a reading of them).
* ``mlp``         -- the gated MLP block the pages' "share of MLP time" refers
  to: the bf16 SwiGLU product Y, then the down projection Z = bf16(Y x W3) with
  fp32 accumulation (Summary, "Problem Statement"; the pages do not spell the
  down projection out, this is the standard gated-MLP reading).

Pins: every function here is checked by ``tests/test_oracle.py`` against fp64
brute force with a closed-form error bound, exact integer regimes, closed
forms of SiLU, a hand-derived rounding table and invariants of the definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]
_lock = threading.Lock()
_default = None


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source file into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP, no fast-math)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    return compile_source(SOURCE, LIB_PATH)


def _u16(x) -> np.ndarray:
    """Accept a numpy uint16 array (bf16 bit patterns) or a torch bf16 tensor."""
    if hasattr(x, "view") and hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch  # only to reinterpret bits; no arithmetic
        x = x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands are passed as uint16 bit patterns, got %s" % a.dtype)
    return a


def _p16(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _pf(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bits -> fp32 values (exact: the bits are the top half of the fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


class Oracle:
    """ctypes view of one compiled oracle library (the default one, or a copy
    the tests compile with a planted mistake to show that the pins catch it)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i64 = ctypes.c_int64
        sig = {
            "oracle_bf16_rne": ([ctypes.c_float], ctypes.c_uint16),
            "oracle_silu": ([ctypes.c_float], ctypes.c_float),
            "oracle_gemm_f32": ([u16p, u16p, i64, i64, i64, f32p], None),
            "oracle_swiglu": ([u16p, u16p, u16p, i64, i64, i64, u16p, f32p, f32p, f32p],
                              ctypes.c_int),
            "oracle_silu_mul": ([u16p, u16p, u16p, i64], None),
            "oracle_gemm_bf16": ([u16p, u16p, i64, i64, i64, u16p], None),
            "oracle_unfused": ([u16p, u16p, u16p, i64, i64, i64, u16p, u16p, u16p], ctypes.c_int),
            "oracle_bf16_rne_array": ([f32p, u16p, i64], None),
            "oracle_silu_array": ([f32p, f32p, i64], None),
            "oracle_e4m3_to_f32": ([ctypes.c_uint8], ctypes.c_float),
            "oracle_swiglu_fp8": ([u8p, u8p, u8p, i64, i64, i64, ctypes.c_float, ctypes.c_float, u16p, f32p],
                                  ctypes.c_int),
            "oracle_set_threads": ([ctypes.c_int], None),
            "oracle_max_threads": ([], ctypes.c_int),
        }
        for name, (argt, rest) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = argt
            fn.restype = rest
        self.lib = lib
        self.path = lib_path

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def bf16_rne(self, p) -> np.ndarray:
        """fp32 -> bf16 bits, round to nearest even, elementwise."""
        arr = np.ascontiguousarray(np.asarray(p, dtype=np.float32))
        out = np.empty(arr.shape, dtype=np.uint16)
        self.lib.oracle_bf16_rne_array(_pf(arr), _p16(out), arr.size)
        return out

    def silu(self, x) -> np.ndarray:
        """SiLU in fp32 through the oracle's own routine, elementwise."""
        arr = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
        out = np.empty(arr.shape, dtype=np.float32)
        self.lib.oracle_silu_array(_pf(arr), _pf(out), arr.size)
        return out

    def gemm_f32(self, A, W) -> np.ndarray:
        """fp32 accumulator of A[M,K] x W[K,N] (bf16 bits in), k increasing."""
        A, W = _u16(A), _u16(W)
        M, K = A.shape
        K2, N = W.shape
        if K2 != K:
            raise ValueError("inner dimensions differ")
        C = np.empty((M, N), dtype=np.float32)
        self.lib.oracle_gemm_f32(_p16(A), _p16(W), M, K, N, _pf(C))
        return C

    def swiglu(self, A, W1, W2, want_p: bool = False, want_gu: bool = False):
        """Y = bf16_RNE(SiLU(A W1) * (A W2)).

        Returns ``Y`` (uint16 bits [M,N]); with ``want_p`` also the fp32 product
        P; with ``want_gu`` also the fp32 Gate and Up accumulators."""
        A, W1, W2 = _u16(A), _u16(W1), _u16(W2)
        M, K = A.shape
        if W1.shape != W2.shape or W1.shape[0] != K:
            raise ValueError("shape mismatch: A %s W1 %s W2 %s" % (A.shape, W1.shape, W2.shape))
        N = W1.shape[1]
        Y = np.empty((M, N), dtype=np.uint16)
        P = np.empty((M, N), dtype=np.float32) if want_p else None
        G = np.empty((M, N), dtype=np.float32) if want_gu else None
        U = np.empty((M, N), dtype=np.float32) if want_gu else None
        rc = self.lib.oracle_swiglu(_p16(A), _p16(W1), _p16(W2), M, K, N, _p16(Y),
                                    _pf(P) if P is not None else None,
                                    _pf(G) if G is not None else None,
                                    _pf(U) if U is not None else None)
        if rc != 0:
            raise RuntimeError("oracle_swiglu failed with code %d" % rc)
        out = [Y]
        if want_p:
            out.append(P)
        if want_gu:
            out += [G, U]
        return out[0] if len(out) == 1 else tuple(out)

    def e4m3_to_f32(self, b) -> np.ndarray:
        """FP8 E4M3 bytes -> fp32 values (exact)."""
        b = np.asarray(b, dtype=np.uint8)
        return np.array([self.lib.oracle_e4m3_to_f32(int(x)) for x in b.ravel()],
                        dtype=np.float32).reshape(b.shape)

    def swiglu_fp8(self, A8, W1_8, W2_8, sg: float, su: float, want_p: bool = False):
        """FP8 variant: Y = bf16_RNE(SiLU(sg * A8 W1_8) * (su * A8 W2_8)),
        E4M3 bytes in, per-tensor scale products sg = fp32(sA*s1), su =
        fp32(sA*s2).  Returns Y (uint16 bits [M,N]), and with ``want_p`` the
        fp32 product P."""
        A8, W1_8, W2_8 = (np.ascontiguousarray(np.asarray(x, dtype=np.uint8)) for x in (A8, W1_8, W2_8))
        M, K = A8.shape
        if W1_8.shape != W2_8.shape or W1_8.shape[0] != K:
            raise ValueError("shape mismatch: A %s W1 %s W2 %s" % (A8.shape, W1_8.shape, W2_8.shape))
        N = W1_8.shape[1]
        Y = np.empty((M, N), dtype=np.uint16)
        P = np.empty((M, N), dtype=np.float32) if want_p else None
        u8p = ctypes.POINTER(ctypes.c_uint8)
        rc = self.lib.oracle_swiglu_fp8(A8.ctypes.data_as(u8p), W1_8.ctypes.data_as(u8p),
                                        W2_8.ctypes.data_as(u8p), M, K, N, float(sg), float(su), _p16(Y),
                                        _pf(P) if P is not None else None)
        if rc != 0:
            raise RuntimeError("oracle_swiglu_fp8 failed with code %d" % rc)
        return (Y, P) if want_p else Y

    def silu_mul(self, Gb, Ub) -> np.ndarray:
        """Elementwise bf16_RNE(SiLU(g) * u) from bf16 Gate and Up."""
        Gb, Ub = _u16(Gb), _u16(Ub)
        if Gb.shape != Ub.shape:
            raise ValueError("shape mismatch")
        Y = np.empty(Gb.shape, dtype=np.uint16)
        self.lib.oracle_silu_mul(_p16(Gb), _p16(Ub), _p16(Y), Gb.size)
        return Y

    def gemm_bf16(self, A, W) -> np.ndarray:
        """bf16_RNE of the fp32 GEMM (one GEMM of the unfused pipeline)."""
        A, W = _u16(A), _u16(W)
        M, K = A.shape
        N = W.shape[1]
        C = np.empty((M, N), dtype=np.uint16)
        self.lib.oracle_gemm_bf16(_p16(A), _p16(W), M, K, N, _p16(C))
        return C

    def mlp(self, A, W1, W2, W3):
        """The gated MLP block: Y = swiglu(A, W1, W2) (bf16), then the down
        projection Z = gemm_bf16(Y, W3), W3 [N, K'].  Returns (Y, Z)."""
        Y = self.swiglu(A, W1, W2)
        return Y, self.gemm_bf16(Y, W3)

    def unfused(self, A, W1, W2):
        """The unfused pipeline: returns (Gate_bf16, Up_bf16, Y)."""
        A, W1, W2 = _u16(A), _u16(W1), _u16(W2)
        M, K = A.shape
        N = W1.shape[1]
        G = np.empty((M, N), dtype=np.uint16)
        U = np.empty((M, N), dtype=np.uint16)
        Y = np.empty((M, N), dtype=np.uint16)
        rc = self.lib.oracle_unfused(_p16(A), _p16(W1), _p16(W2), M, K, N,
                                     _p16(G), _p16(U), _p16(Y))
        if rc != 0:
            raise RuntimeError("oracle_unfused failed with code %d" % rc)
        return G, U, Y


def default() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if missing)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIB_PATH):
                build(force=True)
            _default = Oracle(LIB_PATH)
        return _default


def set_threads(n: int) -> None:
    default().set_threads(n)


def max_threads() -> int:
    return default().max_threads()


def bf16_rne(p) -> np.ndarray:
    return default().bf16_rne(p)


def silu(x) -> np.ndarray:
    return default().silu(x)


def gemm_f32(A, W) -> np.ndarray:
    return default().gemm_f32(A, W)


def swiglu(A, W1, W2, want_p: bool = False, want_gu: bool = False):
    return default().swiglu(A, W1, W2, want_p=want_p, want_gu=want_gu)


def silu_mul(Gb, Ub) -> np.ndarray:
    return default().silu_mul(Gb, Ub)


def gemm_bf16(A, W) -> np.ndarray:
    return default().gemm_bf16(A, W)


def unfused(A, W1, W2):
    return default().unfused(A, W1, W2)


def mlp(A, W1, W2, W3):
    return default().mlp(A, W1, W2, W3)


def e4m3_to_f32(b) -> np.ndarray:
    return default().e4m3_to_f32(b)


def swiglu_fp8(A8, W1_8, W2_8, sg: float, su: float, want_p: bool = False):
    return default().swiglu_fp8(A8, W1_8, W2_8, sg, su, want_p=want_p)
