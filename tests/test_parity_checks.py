"""The fused acceptance checks (tests/parity.py) on the CPU: a result that
is the oracle's own Top-k with fp32-rounded scores passes, and results with a
planted mistake fail: the row's best key swapped for the (k+1)-th, a score off
by 5%, a duplicate index, wrong padding.  Inputs with exact fp32 scores must
match bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from parity import check_fused_exact, check_fused_rows, fp32_score_bound


def _oracle_result(case, extra=1):
    """The oracle's own selection, as a kernel would return it (fp32 scores)."""
    k = case.k
    idx, val, n = oracle.fused_topk(case)
    gi = np.full((case.T, k), -1, np.int32)
    gs = np.full((case.T, k), -np.inf, np.float32)
    for t in range(case.T):
        gi[t, :n[t]] = idx[t, :n[t]]
        gs[t, :n[t]] = val[t, :n[t]].astype(np.float32)
    return gi, gs


@pytest.fixture(scope="module")
def case():
    return synth.gen_fused(6, 8, 64, 3000, 40, q_dtype=synth.BF16, k_dtype=synth.BF16,
                           kv_len=[3000, 2999, 40, 39, 0, 3000 + 5], seed=3)


def test_oracle_selection_passes(case):
    gi, gs = _oracle_result(case)
    rec = check_fused_rows(case, range(case.T), gi, gs)
    assert (rec == 1.0).all()


def test_dropping_the_best_key_fails(case):
    gi, gs = _oracle_result(case)
    t = 0
    row = oracle.fused_score_row(case, t)
    order = np.lexsort((np.arange(row.size), -row))
    gi[t, 0], gs[t, 0] = order[case.k], np.float32(row[order[case.k]])  # (k+1)-th instead of the best
    with pytest.raises(AssertionError, match="left out"):
        check_fused_rows(case, [t], gi, gs, min_recall=None)


@pytest.mark.parametrize("mistake", ["score", "duplicate", "padding"])
def test_planted_mistakes_fail(case, mistake):
    gi, gs = _oracle_result(case)
    if mistake == "score":
        gs[1, 3] *= np.float32(1.05)
    elif mistake == "duplicate":
        gi[1, 3] = gi[1, 4]
    else:
        gi[2, case.k - 1] = 5  # row 2 has 40 valid keys and k = 40: no padding ... use row 3
        gi[3, case.k - 1] = 5
    with pytest.raises(AssertionError):
        check_fused_rows(case, [1, 3], gi, gs)


def test_bound_is_tight_enough_to_matter(case):
    # the fp32 bound is a small fraction of a typical score, so the strict
    # checks constrain the result far below the relative tolerance
    idx, val, n = oracle.fused_topk(case, rows=[0])
    b = fp32_score_bound(case, 0, idx[0, :n[0]])
    assert (b / np.abs(val[0, :n[0]])).max() < 1e-4


@pytest.mark.parametrize("qt,kt,fp8,no_relu,H", [(synth.BF16, synth.BF16, False, False, 8),
                                                 (synth.F16, synth.FP8_E4M3, False, False, 5),
                                                 (synth.BF16, synth.FP8_E4M3, True, False, 64),
                                                 (synth.F16, synth.F16, False, True, 1),
                                                 (synth.F32, synth.F32, False, False, 3)])
def test_exact_family_scores_are_fp32_exact(qt, kt, fp8, no_relu, H):
    """The exact family's scores equal their fp32 rounding (so a kernel's
    fp32 arithmetic reproduces them), ties are frequent, and the oracle's
    own result passes the bit-exact check."""
    D = 256 if H <= 32 else 128
    case = synth.gen_fused_exact(4, H, D, 2000, 100, q_dtype=qt, k_dtype=kt, fp8_score=fp8, no_relu=no_relu,
                                 kv_len=[2000, 1500, 100, 7], seed=H)
    for t in range(case.T):
        row = oracle.fused_score_row(case, t)
        assert np.array_equal(row, row.astype(np.float32).astype(np.float64))
        if row.size >= 1000:
            assert np.unique(row).size < row.size  # ties
    gi, gs = _oracle_result(case)
    check_fused_exact(case, range(case.T), gi, gs)
    gi[0, :2] = gi[0, 1::-1]  # order is free
    gs[0, :2] = gs[0, 1::-1]
    check_fused_exact(case, range(case.T), gi, gs)
    gi[1, 0] = np.setdiff1d(np.arange(1500), gi[1])[0]
    with pytest.raises(AssertionError):
        check_fused_exact(case, [1], gi, gs)
