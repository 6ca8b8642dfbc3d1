"""CPU oracle: plain, slow, obviously correct.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product library never loads it and shares
no code with it; see ``oracle.c`` for the definitions it implements:

* the lightning-indexer score of LiteTopK Sec. 2.1 Eq. (1), summed in double
  over every causally valid key (no blocking, no sampling), with lengths
  clamped to [0, N];
* with the FP8-scoring flag, the same score over queries quantized per
  (query, head) row to e4m3fn (the FP8 indexer of LiteTopK Sec. 2.1; the
  encoder is written from the OCP E4M3 definition), and
* exact Top-k as a full sort by (score descending, index ascending)
  (LiteTopK Sec. 3.1 Eq. (2); Sample-Guided Exact Top-K Sec. 6.1 Eq. (30)).

Pins (tests/test_oracle.py) tie it to things other than itself: exhaustive
format decodes and the e4m3fn encoder over every fp32 bit pattern against
torch/numpy casts, numpy matmul for the H = 1 inner
product, positive-orthant and sign-flip closed forms for ReLU, monotone rows,
brute-force subset enumeration for selection, and the exactness invariants.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from .build import build as _build, LIB_PATH

_lib = None


def _load():
    global _lib
    if _lib is None:
        _build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        P, I, I64, U32, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double
        lib.ora_decode.argtypes = [I, U32]
        lib.ora_decode.restype = D
        lib.ora_decode_array.argtypes = [I, P, P, I64]
        lib.ora_encode_e4m3.argtypes = [ctypes.c_float]
        lib.ora_encode_e4m3.restype = ctypes.c_uint8
        lib.ora_encode_e4m3_array.argtypes = [P, P, I64, I]
        lib.ora_select_f64.argtypes = [P, I64, I, P, P]
        lib.ora_select_f64.restype = I
        lib.ora_select_f32.argtypes = [P, I64, I, P]
        lib.ora_select_f32.restype = I
        lib.ora_fused_topk.argtypes = [P, I, P, I, P, P, P, I64, I, I, U32, P, I, I, P, P, P, I]
        lib.ora_fused_topk.restype = I
        lib.ora_fused_scores_at.argtypes = [P, I, P, I, P, P, I64, I, I, U32, P, P, I64, P]
        lib.ora_fused_scores_at.restype = I
        lib.ora_fused_score_row.argtypes = [P, I, P, I, P, P, I64, I, I, U32, I, I64, P]
        lib.ora_fused_score_row.restype = I64
        lib.ora_topk_ragged.argtypes = [P, I64, P, P, I, I, P, P, I]
        lib.ora_prior_from_topk.argtypes = [P, I64, I, I64, I, P]
        lib.ora_prior_from_topk.restype = I
        lib.ora_topk_ragged.restype = I
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Widen raw bits (float32 / uint16 / uint8 arrays) to float64."""
    src = np.ascontiguousarray(bits)
    out = np.empty(src.shape, dtype=np.float64)
    _load().ora_decode_array(dtype, _ptr(src), _ptr(out), src.size)
    return out


def encode_e4m3(x: np.ndarray, nthreads: Optional[int] = None) -> np.ndarray:
    """e4m3fn codes (uint8) of float32 values: nearest value, ties to even;
    NaN (0x7F, sign kept) for NaN, inf and magnitudes that round above 448."""
    src = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(src.shape, dtype=np.uint8)
    _load().ora_encode_e4m3_array(_ptr(src), _ptr(out), src.size, nthreads or default_threads())
    return out


def valid_len(case, t: int) -> int:
    """L_t = min(max(kv_len[t], 0), N)."""
    return int(min(max(int(case.kv_len[t]), 0), case.N))


def select(row: np.ndarray, k: int):
    """Exact Top-k of one row: indices sorted by (value desc, index asc).

    Returns (idx[k] int32 padded with -1, n = min(k, L)); for float64 rows also
    the selected values (padded with -inf)."""
    row = np.ascontiguousarray(row)
    idx = np.empty(k, dtype=np.int32)
    lib = _load()
    if row.dtype == np.float64:
        val = np.empty(k, dtype=np.float64)
        n = lib.ora_select_f64(_ptr(row), row.size, k, _ptr(idx), _ptr(val))
        if n < 0:
            raise RuntimeError(f"ora_select_f64 failed: {n}")
        return idx, n, val
    row = row.astype(np.float32, copy=False)
    n = lib.ora_select_f32(_ptr(row), row.size, k, _ptr(idx))
    if n < 0:
        raise RuntimeError(f"ora_select_f32 failed: {n}")
    return idx, n


def _fused_arrays(case):
    Q = np.ascontiguousarray(case.q_bits)
    K = np.ascontiguousarray(case.k_bits)
    S = None if case.k_scale is None else np.ascontiguousarray(case.k_scale, dtype=np.float32)
    W = np.ascontiguousarray(case.W, dtype=np.float32)
    return Q, K, S, W


def fused_topk(case, rows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """Oracle Top-k of the fused score for ``rows`` (default: all queries).

    Returns (idx [R, k] int32, score [R, k] float64, n [R] int32), each row
    sorted by (score desc, index asc) and padded with (-1, -inf)."""
    rows = np.arange(case.T, dtype=np.int32) if rows is None else np.asarray(rows, dtype=np.int32)
    Q, K, S, W = _fused_arrays(case)
    kv = np.ascontiguousarray(case.kv_len, dtype=np.int32)
    R = rows.size
    idx = np.empty((R, case.k), dtype=np.int32)
    val = np.empty((R, case.k), dtype=np.float64)
    n = np.empty(R, dtype=np.int32)
    rc = _load().ora_fused_topk(_ptr(Q), case.q_dtype, _ptr(K), case.k_dtype, _ptr(S), _ptr(W),
                                _ptr(kv), case.N, case.H, case.D, case.flags, _ptr(rows), R, case.k,
                                _ptr(idx), _ptr(val), _ptr(n), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ora_fused_topk failed: {rc}")
    return idx, val, n


def fused_score_row(case, t: int, L: Optional[int] = None) -> np.ndarray:
    """The full float64 score row of query ``t`` over keys [0, L), L clamped
    to [0, N] (default: kv_len[t])."""
    L = int(case.kv_len[t]) if L is None else int(L)
    Q, K, S, W = _fused_arrays(case)
    out = np.empty(max(0, min(L, case.N)), dtype=np.float64)
    rc = _load().ora_fused_score_row(_ptr(Q), case.q_dtype, _ptr(K), case.k_dtype, _ptr(S), _ptr(W),
                                     case.N, case.H, case.D, case.flags, int(t), L, _ptr(out))
    if rc != out.size:
        raise RuntimeError(f"ora_fused_score_row failed: {rc}")
    return out


def fused_scores_at(case, t_idx, j_idx) -> np.ndarray:
    """Scores of individual (query, key) pairs."""
    t_idx = np.ascontiguousarray(t_idx, dtype=np.int32)
    j_idx = np.ascontiguousarray(j_idx, dtype=np.int64)
    Q, K, S, W = _fused_arrays(case)
    out = np.empty(t_idx.size, dtype=np.float64)
    rc = _load().ora_fused_scores_at(_ptr(Q), case.q_dtype, _ptr(K), case.k_dtype, _ptr(S), _ptr(W),
                                     case.N, case.H, case.D, case.flags, _ptr(t_idx), _ptr(j_idx), t_idx.size,
                                     _ptr(out))
    if rc != 0:
        raise RuntimeError(f"ora_fused_scores_at failed: {rc}")
    return out


def topk_ragged(case, rows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """Oracle Top-k of the listed rows of a ragged fp32 score matrix.

    Returns (idx [R, k] int32 sorted by (value desc, index asc), n [R])."""
    rows = np.arange(case.M, dtype=np.int32) if rows is None else np.asarray(rows, dtype=np.int32)
    X = np.ascontiguousarray(case.scores, dtype=np.float32)
    rl = np.ascontiguousarray(case.row_len, dtype=np.int32)
    R = rows.size
    idx = np.empty((R, case.k), dtype=np.int32)
    n = np.empty(R, dtype=np.int32)
    rc = _load().ora_topk_ragged(_ptr(X), case.pitch, _ptr(rl), _ptr(rows), R, case.k,
                                 _ptr(idx), _ptr(n), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"ora_topk_ragged failed: {rc}")
    return idx, n


def prior_from_topk(prev_idx: np.ndarray, N: int, k_prime: int) -> np.ndarray:
    """History sample (LiteTopK Sec. 3.2 "Sampling"): the ``k_prime`` keys
    that occur most often in the previous chunk's Top-k lists ``prev_idx``
    [T_prev, k] (count descending, index ascending; entries outside [0, N)
    ignored), padded with -1 past min(k_prime, N), in that order."""
    prev = np.ascontiguousarray(prev_idx, dtype=np.int32)
    if prev.ndim != 2:
        raise ValueError("prev_idx must be [T_prev, k]")
    out = np.empty(k_prime, dtype=np.int32)
    n = _load().ora_prior_from_topk(_ptr(prev), prev.shape[0], prev.shape[1], N, k_prime, _ptr(out))
    if n < 0:
        raise RuntimeError(f"ora_prior_from_topk failed ({n})")
    return out
