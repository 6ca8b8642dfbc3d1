"""Acceptance checks of HIP results against the CPU oracle (test helpers).

Fused path (scores differ from the oracle only by fp32 accumulation order):
  (i)   every returned score is within tol of the oracle score of its index,
        relative to max(|oracle score|, |oracle k-th score|);
  (ii)  every returned index's oracle score >= oracle k-th score - tol*|k-th|;
  (iii) |out| = min(k, L), indices distinct and in [0, L), padding -1 / -inf;
  (iv)  recall |S_gpu & S_oracle| / min(k, L) is reported.
Standalone path: the index sets are bit-exact.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = {0: 2e-2, 1: 2e-2, 2: 2e-2, 3: 6e-2}  # by key dtype: f32, bf16, f16, fp8


def check_fused_rows(case, rows, gpu_idx, gpu_score, tol=None, min_recall=None):
    """Check rows ``rows`` of a fused result; returns the per-row recalls."""
    tol = TOL[case.k_dtype] if tol is None else tol
    rows = np.asarray(rows, dtype=np.int32)
    o_idx, o_val, o_n = oracle.fused_topk(case, rows=rows)
    recalls = []
    for r, t in enumerate(rows):
        L = int(case.kv_len[t])
        need = min(case.k, max(L, 0))
        gi = np.asarray(gpu_idx[t])
        gs = np.asarray(gpu_score[t])
        assert o_n[r] == need
        assert (gi[need:] == -1).all(), f"row {t}: padding indices"
        assert np.isneginf(gs[need:]).all(), f"row {t}: padding scores"
        sel = gi[:need]
        assert len(np.unique(sel)) == need, f"row {t}: duplicate indices"
        assert ((sel >= 0) & (sel < L)).all(), f"row {t}: index out of range"
        if need == 0:
            recalls.append(1.0)
            continue
        kth = o_val[r, need - 1]
        ora_sel = oracle.fused_scores_at(case, np.full(need, t), sel)
        # relative to max(|own score|, |k-th score|, 1e-3 |top score|): the
        # last term keeps near-zero scores of rows whose k-th score is 0
        # (fewer valid keys than k, ReLU zeros) at the row's scale, where fp32
        # accumulation-order differences are absolute, not relative
        denom = np.maximum(np.maximum(np.abs(ora_sel), abs(kth)), 1e-3 * abs(o_val[r, 0]))
        denom = np.where(denom > 0, denom, 1.0)
        err = np.abs(gs[:need].astype(np.float64) - ora_sel) / denom
        assert err.max() <= tol, f"row {t}: score error {err.max():.3g} > {tol}"
        assert (ora_sel >= kth - tol * abs(kth)).all(), \
            f"row {t}: selected score {ora_sel.min():.6g} below k-th {kth:.6g}"
        rec = len(set(sel.tolist()) & set(o_idx[r, :need].tolist())) / need
        recalls.append(rec)
    recalls = np.asarray(recalls)
    if min_recall is not None:
        assert recalls.min() >= min_recall, f"recall {recalls.min():.4f} < {min_recall}"
    return recalls


def check_ragged_exact(case, gpu_idx, rows=None):
    rows = np.arange(case.M) if rows is None else np.asarray(rows)
    o_idx, o_n = oracle.topk_ragged(case, rows=rows)
    for r, m in enumerate(rows):
        need = int(o_n[r])
        gi = np.asarray(gpu_idx[m])
        assert (gi[need:] == -1).all(), f"row {m}: padding"
        got = np.sort(gi[:need])
        exp = np.sort(o_idx[r, :need])
        if not np.array_equal(got, exp):
            miss = np.setdiff1d(exp, got)[:8]
            extra = np.setdiff1d(got, exp)[:8]
            raise AssertionError(f"row {m} (L={case.row_len[m]}): missing {miss.tolist()} extra {extra.tolist()}")


def fp8_score_bound(case, t, idx):
    """Bound on |score - exact score| when query row (t, h) is quantized to
    e4m3fn with scale s_h = max|q[t,h,:]| / 448 (round to nearest even):
    each element moves by at most 2^-4 of itself (3 mantissa bits) or, below
    the normal range, by 2^-10 s_h; ReLU is 1-Lipschitz, so
        |ds| <= sum_h |w_h| sum_d (2^-4 |q_hd| + 2^-10 s_h) |k_d|,
    plus fp32 accumulation (covered by a 10% margin)."""
    q = oracle.decode(case.q_bits[t], case.q_dtype).reshape(case.H, case.D)
    k = oracle.decode(case.k_bits[np.asarray(idx)], case.k_dtype).reshape(len(idx), case.D)
    if case.k_scale is not None:
        k = k * case.k_scale[np.asarray(idx)].astype(np.float64)[:, None]
    s = np.abs(q).max(axis=1) / 448.0
    w = np.abs(case.W[t].astype(np.float64))
    ak = np.abs(k)
    per_head = (2.0 ** -4) * (np.abs(q) @ ak.T) + (2.0 ** -10) * s[:, None] * ak.sum(axis=1)[None, :]
    return 1.1 * (w[:, None] * per_head).sum(axis=0)


def check_fp8_score_rows(case, rows, gpu_idx, gpu_score, min_recall=None):
    """FP8-scoring results: invariants, each returned score within the
    quantization bound of its exact score, and no returned index whose exact
    score lies further below the exact k-th score than the two bounds allow."""
    rows = np.asarray(rows, dtype=np.int32)
    o_idx, o_val, o_n = oracle.fused_topk(case, rows=rows)
    recalls = []
    for r, t in enumerate(rows):
        L = int(case.kv_len[t])
        need = min(case.k, max(L, 0))
        gi, gs = np.asarray(gpu_idx[t]), np.asarray(gpu_score[t])
        assert o_n[r] == need
        assert (gi[need:] == -1).all() and np.isneginf(gs[need:]).all(), f"row {t}: padding"
        sel = gi[:need]
        assert len(np.unique(sel)) == need and ((sel >= 0) & (sel < L)).all(), f"row {t}: invalid indices"
        if need == 0:
            recalls.append(1.0)
            continue
        ora_sel = oracle.fused_scores_at(case, np.full(need, t), sel)
        b_sel = fp8_score_bound(case, t, sel)
        err = np.abs(gs[:need].astype(np.float64) - ora_sel)
        assert (err <= b_sel).all(), f"row {t}: score error {(err / b_sel).max():.3g} x the bound"
        kth = o_val[r, need - 1]
        b_ora = fp8_score_bound(case, t, o_idx[r, :need])
        assert (ora_sel >= kth - b_sel - b_ora.max()).all(), f"row {t}: a selected score is too low"
        recalls.append(len(set(sel.tolist()) & set(o_idx[r, :need].tolist())) / need)
    recalls = np.asarray(recalls)
    if min_recall is not None:
        assert recalls.min() >= min_recall, f"recall {recalls.min():.4f} < {min_recall}"
    return recalls
