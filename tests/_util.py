"""Shared helpers for the GPU parity tests (comparison rules, oracle sampling,
and a disk cache of whole-tensor oracle results)."""
import hashlib
import os
import sys

import numpy as np
import torch

import oracle
from swiglu_gated_mlp_amd import inputs

ATOL = 1e-3
RTOL = 8e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f32(bits):
    return oracle.bf16_to_f32(bits)


def gpu_bits(y: torch.Tensor) -> np.ndarray:
    return inputs.as_bits(y.cpu())


def check_close(got_bits, ref_bits, what=""):
    """Acceptance rule: |y - ref| <= 1e-3 + 8e-3 |ref| for every element, with
    y the GPU's bf16 and ref the oracle's bf16 (both widened to fp32)."""
    got = f32(got_bits).astype(np.float64)
    ref = f32(ref_bits).astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_ok = np.isnan(got) == np.isnan(ref)
    assert nan_ok.all(), "%s: NaN pattern differs" % what
    err = np.abs(got - ref)
    lim = ATOL + RTOL * np.abs(ref)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, "%s: %d elements outside tolerance, first at %s got %r want %r" % (
        what, len(bad), bad[0].tolist(), got[tuple(bad[0])], ref[tuple(bad[0])])


def mismatch_rates(got_bits, ref_bits, ref_p=None):
    """(bitwise bf16 mismatch rate, fraction with >1% relative error vs fp32 P)."""
    g = np.asarray(got_bits)
    r = np.asarray(ref_bits)
    same = (g == r) | (((g | r) & 0x7FFF) == 0)     # +0 == -0
    bitwise = 1.0 - same.mean()
    page = None
    if ref_p is not None:
        gv = f32(g).astype(np.float64)
        page = float((np.abs(gv - ref_p) > 0.01 * np.abs(ref_p)).mean())
    return float(bitwise), page


def sample_rows(M, n=6):
    rows = sorted(set([0, M - 1] + list(np.linspace(0, M - 1, n).astype(int))))
    return [r for r in rows if 0 <= r < M]


def sample_cols(N, n=12, tile=128):
    cols = set([0, N - 1, tile - 1, min(N - 1, tile)])
    cols.update(np.linspace(0, N - 1, n).astype(int).tolist())
    return sorted(c for c in cols if 0 <= c < N)


def oracle_rows(A, W1, W2, rows, want_p=False):
    return oracle.swiglu(A[rows].contiguous(), W1, W2, want_p=want_p)


def oracle_cols(A, W1, W2, cols, want_p=False):
    return oracle.swiglu(A, W1[:, cols].contiguous(), W2[:, cols].contiguous(), want_p=want_p)


# ---------------------------------------------------------------------------
# every-element comparison of large outputs
# ---------------------------------------------------------------------------

def diff_positions(got_bits, ref_bits):
    """Flat indices where the bf16 bit patterns differ (+0 and -0 count as
    equal).  Every other element is exactly the oracle's value."""
    g = np.ascontiguousarray(got_bits).reshape(-1)
    r = np.ascontiguousarray(ref_bits).reshape(-1)
    idx = np.flatnonzero(g != r)
    if idx.size:
        zero = ((g[idx] | r[idx]) & 0x7FFF) == 0
        idx = idx[~zero]
    return idx


def check_close_all(got_bits, ref_bits, what=""):
    """check_close over every element, evaluated only where the bits differ
    (identical bits always meet the rule).  Returns the differing indices."""
    assert np.shape(got_bits) == np.shape(ref_bits), (np.shape(got_bits), np.shape(ref_bits))
    idx = diff_positions(got_bits, ref_bits)
    if idx.size:
        g = np.ascontiguousarray(got_bits).reshape(-1)[idx]
        r = np.ascontiguousarray(ref_bits).reshape(-1)[idx]
        try:
            check_close(g, r, what)
        except AssertionError as e:
            first = np.unravel_index(int(idx[0]), np.shape(ref_bits))
            raise AssertionError("%s (first differing element at %s)" % (e, list(map(int, first))))
    return idx


class PageMetric:
    """The pages' mismatch metric, the share of elements with more than 1 %
    relative error against the oracle's fp32 product P, over every element.
    The oracle's own bf16 Y is scored once; a GPU result then only needs its
    differing elements re-scored."""

    def __init__(self, ref_bits, P):
        self.ref = np.ascontiguousarray(ref_bits).reshape(-1)
        self.P = np.ascontiguousarray(P, dtype=np.float32).reshape(-1)
        self.n = self.ref.size
        self.base = np.empty(self.n, dtype=bool)
        step = 1 << 24
        for a in range(0, self.n, step):
            p = self.P[a:a + step].astype(np.float64)
            y = f32(self.ref[a:a + step]).astype(np.float64)
            self.base[a:a + step] = np.abs(y - p) > 0.01 * np.abs(p)
        self.base_count = int(self.base.sum())

    def rates(self, idx, got_bits):
        """(bitwise mismatch rate, > 1 % rate) for a result differing from the
        oracle's Y at flat indices idx."""
        if self.n == 0:
            return 0.0, 0.0
        g = np.ascontiguousarray(got_bits).reshape(-1)[idx]
        p = self.P[idx].astype(np.float64)
        hit = np.abs(f32(g).astype(np.float64) - p) > 0.01 * np.abs(p)
        count = self.base_count - int(self.base[idx].sum()) + int(hit.sum())
        return idx.size / self.n, count / self.n


# ---------------------------------------------------------------------------
# whole-tensor oracle results, cached on disk (git-ignored build/), keyed by
# a label, the oracle's source and the input generator's source
# ---------------------------------------------------------------------------
_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CACHE_DIR = os.path.join(_ROOT, "build", "oracle_cache")


def _sources_digest():
    h = hashlib.sha256()
    for rel in ("oracle/oracle.c", "oracle/__init__.py", "swiglu_gated_mlp_amd/inputs.py"):
        with open(os.path.join(_ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cached_oracle(label, compute, want_p=False):
    """compute() -> Y bits (or (Y, P) when want_p), loaded from the cache when
    an earlier run stored it for the same label and sources.  A cache that
    cannot be written (read-only or full disk) is skipped."""
    stem = os.path.join(CACHE_DIR, "%s-%s" % (label, _sources_digest()))
    names = [stem + ".Y.npy"] + ([stem + ".P.npy"] if want_p else [])
    if all(os.path.exists(n) for n in names):
        try:
            arrs = [np.load(n) for n in names]
            return tuple(arrs) if want_p else arrs[0]
        except (OSError, ValueError):
            pass
    out = compute()
    arrs = list(out) if want_p else [out]
    try:
        os.makedirs(CACHE_DIR, exist_ok=True)
        for n, a in zip(names, arrs):
            tmp = n + ".tmp%d.npy" % os.getpid()
            np.save(tmp, a)
            os.replace(tmp, n)
    except OSError:
        pass
    return out
