"""Acceptance checks of HIP results against the CPU oracle (test helpers).

Fused path.  The kernel selects the exact Top-k of its own fp32 scores, and
its scores differ from the oracle's double-precision scores only by fp32
rounding.  For each checked row, with s the oracle score, s_k the oracle's
k-th score, need = min(k, L) and tol the relative tolerance of the key dtype:

  (i)   invariants: |out| = need, indices distinct and in [0, L), padding
        -1 / -inf past need;
  (ii)  every returned score is within max(tol * max(|s_j|, |s_k|), B_j) of
        the oracle score of its index;
  (iii) every returned index j has s_j >= s_k - max(tol * |s_k|, B_j + B*);
  (iv)  every index of the oracle's Top-k that was not returned has
        s_i <= s_k + max(tol * |s_k|, B_i + B*);
  (v)   recall |S_gpu & S_oracle| / need is reported, and its mean over the
        checked rows must reach min_recall.

B_j is a derived bound on the fp32 rounding of key j's score (see
``fp32_score_bound``) and B* its maximum over the returned keys and the
oracle's Top-k.  With ``strict`` (the default) the checks are also made
without the relative tolerance: |gpu_j - s_j| <= B_j, s_j >= s_k - (B_j + B*)
and s_i <= s_k + (B_i + B*).  These follow from exact selection on scores
within B of the oracle's: if the kernel returned j over an oracle Top-k key i,
then gpu_j >= gpu_i, so s_j + B_j >= s_i - B_i.

``check_fused_exact`` is the bar for inputs whose scores are exact in fp32
(small integers, power-of-two weights and scales): the index sets and the
scores must equal the oracle's bit for bit.

Standalone path: the index sets are bit-exact.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = {0: 2e-2, 1: 2e-2, 2: 2e-2, 3: 6e-2}  # by key dtype: f32, bf16, f16, fp8

# unit roundoff of a faithful fp32 rounding (2^-23 also covers directed
# rounding inside the matrix cores)
U32 = 2.0 ** -23


def _decoded_query(case, t):
    """Query t as the kernel multiplies it: [H, D] float64, and the per-head
    factor folded into the weight (the FP8 scale when queries are quantized)."""
    q = synth.decode_reference_free(np.ascontiguousarray(case.q_bits[t]), case.q_dtype).astype(np.float64)
    q = q.reshape(case.H, case.D)
    fac = np.ones(case.H)
    if case.flags & 2:  # FP8 scoring: the oracle's quantization (codes and scales)
        amax = np.abs(q).max(axis=1).astype(np.float32)
        ok = (amax > 0) & np.isfinite(amax)
        inv = np.where(ok, np.float32(448.0) / np.where(ok, amax, 1), 0).astype(np.float32)
        codes = oracle.encode_e4m3((q.astype(np.float32) * inv[:, None]).astype(np.float32))
        q = oracle.decode(codes, synth.FP8_E4M3)
        fac = np.where(ok, (amax / np.float32(448.0)).astype(np.float32), 1.0).astype(np.float64)
    return q, fac


def fp8_mfma_alignment_error(p):
    """Bound on what the FP8 matrix cores lose when they sum the products
    ``p`` [..., D] (unscaled e4m3fn x e4m3fn, D a multiple of 64) of one dot
    product.  The scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) does not
    round like an fp32 sum: it adds each group of 8 consecutive products
    aligned to the group's largest, truncating every product toward zero to
    a multiple of 2^(E - 13) (E the exponent of the group's largest |p|), and
    the group sums at fp32 precision (tests/test_probe_gpu.py pins this).  So
    each of the 7 other products of a group loses less than 2^(E - 13)."""
    p = np.abs(np.asarray(p, dtype=np.float64))
    g = p.reshape(p.shape[:-1] + (p.shape[-1] // 8, 8)).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(g > 0, np.floor(np.log2(np.where(g > 0, g, 1.0))), -np.inf)
    return (7.0 * np.exp2(e - 13.0)).sum(axis=-1)


def fp32_score_bound(case, t, idx):
    """Bound on |fp32 score - exact score| of keys ``idx`` of query t.

    The kernel forms each head's dot product over D terms in fp32 (the
    products of 16-bit or FP8 operands are exact), applies the ReLU
    (1-Lipschitz), accumulates w_h * ReLU(dot_h) over H heads with one
    rounding per step, and applies at most four more roundings (half-wave
    combine, per-key scale, folded weight scale, final product).  By the
    standard bound on a recursive sum, |error| <= gamma_n * A with
    n = D + H + 8, gamma_n = n u / (1 - n u) and
    A = sum_h |w_h f_h| sum_d |q_hd k_jd| (the magnitude of every term).
    With FP8 scoring the dot products come from the FP8 matrix cores, whose
    in-group alignment (``fp8_mfma_alignment_error``) adds
    sum_h |w_h f_h| s_j align_h(q8_h * k8_j) on top (s_j the key's scale)."""
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size == 0:
        return np.zeros(0)
    q, fac = _decoded_query(case, t)
    k = synth.decode_reference_free(np.ascontiguousarray(case.k_bits[idx]), case.k_dtype).astype(np.float64)
    k = k.reshape(idx.size, case.D)
    if case.k_scale is not None:
        k = k * np.abs(case.k_scale[idx].astype(np.float64))[:, None]
    w = np.abs(case.W[t].astype(np.float64)) * fac
    A = w @ (np.abs(q) @ np.abs(k).T)
    n = case.D + case.H + 8
    gamma = n * U32 / (1.0 - n * U32)
    bound = gamma * A
    if case.flags & 2:  # FP8 scoring: the matrix cores' in-group alignment
        k8 = synth.decode_reference_free(np.ascontiguousarray(case.k_bits[idx]), case.k_dtype).astype(np.float64)
        k8 = k8.reshape(idx.size, case.D)
        scale = np.abs(case.k_scale[idx].astype(np.float64)) if case.k_scale is not None else np.ones(idx.size)
        for c0 in range(0, idx.size, 256):  # [keys, H, D] products, a chunk of keys at a time
            prod = k8[c0:c0 + 256, None, :] * q[None, :, :]
            bound[c0:c0 + 256] += (fp8_mfma_alignment_error(prod) @ w) * scale[c0:c0 + 256]
    return bound


def _row_checks(case, t, gi, gs, o_idx_row, o_val_row, o_n, tol, strict):
    L = oracle.valid_len(case, t)
    need = min(case.k, L)
    assert o_n == need, f"row {t}: oracle count {o_n} != {need}"
    assert (gi[need:] == -1).all(), f"row {t}: padding indices"
    assert np.isneginf(gs[need:]).all(), f"row {t}: padding scores"
    sel = gi[:need]
    assert len(np.unique(sel)) == need, f"row {t}: duplicate indices"
    assert ((sel >= 0) & (sel < L)).all(), f"row {t}: index out of range"
    if need == 0:
        return 1.0
    kth = o_val_row[need - 1]
    top = o_idx_row[:need]
    ora_sel = oracle.fused_scores_at(case, np.full(need, t), sel)
    missed = np.setdiff1d(top, sel)
    ora_missed = oracle.fused_scores_at(case, np.full(missed.size, t), missed) if missed.size else np.zeros(0)
    b_sel = fp32_score_bound(case, t, sel)
    b_top = fp32_score_bound(case, t, top)
    b_missed = fp32_score_bound(case, t, missed)
    bstar = max(b_sel.max(), b_top.max())
    got = gs[:need].astype(np.float64)
    err = np.abs(got - ora_sel)
    rel = np.maximum(np.abs(ora_sel), abs(kth))
    assert (err <= np.maximum(tol * rel, b_sel)).all(), \
        f"row {t}: score error {np.max(err / np.maximum(tol * rel, b_sel)):.3g} x the tolerance"
    assert (ora_sel >= kth - np.maximum(tol * abs(kth), b_sel + bstar)).all(), \
        f"row {t}: a returned score {ora_sel.min():.8g} lies below the k-th {kth:.8g}"
    assert (ora_missed <= kth + np.maximum(tol * abs(kth), b_missed + bstar)).all(), \
        f"row {t}: a Top-k key left out scores {ora_missed.max():.8g} above the k-th {kth:.8g}"
    if strict:
        assert (err <= b_sel).all(), f"row {t}: score error {np.max(err / np.maximum(b_sel, 1e-300)):.3g} x the fp32 bound"
        assert (ora_sel >= kth - (b_sel + bstar)).all(), f"row {t}: returned score below the k-th beyond the fp32 bound"
        assert (ora_missed <= kth + (b_missed + bstar)).all(), f"row {t}: Top-k key left out beyond the fp32 bound"
    return (need - missed.size) / need


def check_fused_rows(case, rows, gpu_idx, gpu_score, tol=None, min_recall=0.99, strict=True, oracle_result=None):
    """Check rows ``rows`` of a fused result (module docstring); returns the
    per-row recalls.  ``min_recall`` bounds their mean.  ``oracle_result``
    may pass oracle.fused_topk(case, rows) when the caller already has it."""
    tol = TOL[case.k_dtype] if tol is None else tol
    rows = np.asarray(list(rows), dtype=np.int32)
    o_idx, o_val, o_n = oracle.fused_topk(case, rows=rows) if oracle_result is None else oracle_result
    recalls = np.array([
        _row_checks(case, int(t), np.asarray(gpu_idx[t]), np.asarray(gpu_score[t]), o_idx[r], o_val[r], int(o_n[r]),
                    tol, strict)
        for r, t in enumerate(rows)])
    if min_recall is not None and recalls.size:
        assert recalls.mean() >= min_recall, f"mean recall {recalls.mean():.4f} < {min_recall}"
    return recalls


def check_fused_exact(case, rows, gpu_idx, gpu_score):
    """Inputs with fp32-exact scores: the returned sets and scores equal the
    oracle's exactly (ties to the lower index included)."""
    rows = np.asarray(list(rows), dtype=np.int32)
    o_idx, o_val, o_n = oracle.fused_topk(case, rows=rows)
    for r, t in enumerate(rows):
        need = int(o_n[r])
        gi, gs = np.asarray(gpu_idx[t]), np.asarray(gpu_score[t])
        assert need == min(case.k, oracle.valid_len(case, int(t)))
        assert (gi[need:] == -1).all() and np.isneginf(gs[need:]).all(), f"row {t}: padding"
        order = np.argsort(gi[:need], kind="stable")
        got_i, got_s = gi[:need][order], gs[:need][order].astype(np.float64)
        o = np.argsort(o_idx[r, :need], kind="stable")
        exp_i, exp_s = o_idx[r, :need][o], o_val[r, :need][o]
        if not np.array_equal(got_i, exp_i):
            miss = np.setdiff1d(exp_i, got_i)[:6]
            extra = np.setdiff1d(got_i, exp_i)[:6]
            raise AssertionError(f"row {t} (L={oracle.valid_len(case, int(t))}, k-th {o_val[r, need - 1]}): "
                                 f"missing {miss.tolist()} extra {extra.tolist()}")
        assert np.array_equal(got_s, exp_s), f"row {t}: scores differ from the exact scores"


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
