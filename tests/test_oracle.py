"""Pins for the CPU oracle (runs without a GPU).

Each test ties the oracle to something other than itself, chosen so that a
plausible mistake (a dropped head or dimension, a wrong sign in the ReLU, a
transposed operand, per-head instead of per-query weights, a wrong tie rule,
ignoring the causal length) fails at least one of them:

* exhaustive decode of every bf16 / fp16 / e4m3fn code against torch/numpy;
* H = 1 without ReLU against numpy's matmul (LiteTopK Sec. 3.1, k-NN case);
* the ReLU score on the positive orthant, where ReLU is the identity and the
  score collapses to a weighted matmul (LiteTopK Sec. 2.1 Eq. (1));
* heads whose query is negated on the positive orthant contribute nothing;
* positive homogeneity of the ReLU score in the per-key FP8 scale;
* a monotone closed form whose Top-k is the last k valid keys;
* selection against brute-force enumeration of all subsets on tiny rows, the
  exactness criterion (Sample-Guided Exact Top-K Sec. 6.1 Eq. (30)) and
  numpy's lexsort.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth


# ----------------------------------------------------------------- decoders
@pytest.mark.parametrize("dtype,nbits", [(synth.BF16, 16), (synth.F16, 16), (synth.FP8_E4M3, 8)])
def test_decode_exhaustive_against_library_casts(dtype, nbits):
    codes = np.arange(1 << nbits, dtype=np.uint16 if nbits == 16 else np.uint8)
    ours = oracle.decode(codes, dtype)
    ref = synth.decode_reference_free(codes, dtype).astype(np.float64)
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ref]))


def test_decode_e4m3fn_landmarks():
    # OCP E4M3: 0x7E = 448 (largest finite), 0x08 = 2^-6 (smallest normal),
    # 0x01 = 2^-9 (smallest subnormal), 0x7F and 0xFF are NaN, 0x38 = 1.0.
    v = oracle.decode(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8], dtype=np.uint8), synth.FP8_E4M3)
    assert list(v) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0]
    assert np.isnan(oracle.decode(np.array([0x7F, 0xFF], dtype=np.uint8), synth.FP8_E4M3)).all()


def _case(T, H, D, N, k, *, q=None, kk=None, W=None, kv_len=None, q_dtype=synth.F32,
          k_dtype=synth.F32, k_scale=None, no_relu=False):
    rng = np.random.default_rng(7)
    q = rng.standard_normal((T, H, D)).astype(np.float32) if q is None else q.astype(np.float32)
    kk = rng.standard_normal((N, D)).astype(np.float32) if kk is None else kk.astype(np.float32)
    W = rng.random((T, H)).astype(np.float32) if W is None else W.astype(np.float32)
    kvl = np.full(T, N, np.int32) if kv_len is None else np.asarray(kv_len, np.int32)
    return synth.FusedCase(name="pin", T=T, H=H, D=D, N=N, k=k, q_dtype=q_dtype, k_dtype=k_dtype,
                           q_bits=synth.encode(q, q_dtype), k_bits=synth.encode(kk, k_dtype),
                           k_scale=k_scale, W=W, kv_len=kvl,
                           flags=synth.FLAG_NO_RELU if no_relu else 0)


def _all_rows(case):
    return np.stack([oracle.fused_score_row(case, t, case.N) for t in range(case.T)])


# ------------------------------------------------------------ score pins
def test_score_against_python_loops():
    """Eq. (1) written out as float64 loops on tiny signed inputs, with some
    negative head weights and causal lengths below N: every score of every
    valid key, to fp32 rounding of the row's magnitude."""
    rng = np.random.default_rng(12)
    T, H, D, N = 3, 3, 8, 40
    q = rng.standard_normal((T, H, D))
    kk = rng.standard_normal((N, D))
    W = rng.random((T, H)) - 0.25
    kv = [40, 23, 1]
    c = _case(T, H, D, N, 5, q=q, kk=kk, W=W, kv_len=kv)
    qf, kf, wf = (c.q_bits.astype(np.float64), c.k_bits.astype(np.float64), c.W.astype(np.float64))
    for t in range(T):
        got = oracle.fused_score_row(c, t)
        assert got.shape == (kv[t],)
        ref = []
        for j in range(kv[t]):
            acc = 0.0
            for h in range(H):
                dot = 0.0
                for d in range(D):
                    dot += qf[t, h, d] * kf[j, d]
                acc += wf[t, h] * max(dot, 0.0)
            ref.append(acc)
        ref = np.array(ref)
        scale = sum(abs(wf[t, h]) * np.abs(qf[t, h]) @ np.abs(kf[j]) for h in range(H) for j in range(kv[t]))
        assert np.max(np.abs(got - ref)) <= 1e-6 * scale / kv[t] + 1e-30


def test_inner_product_equals_numpy_matmul():
    c = _case(5, 1, 24, 37, 4, W=np.ones((5, 1)), no_relu=True)
    q = c.q_bits.reshape(5, 24).astype(np.float64)
    ref = q @ c.k_bits.astype(np.float64).T
    np.testing.assert_allclose(_all_rows(c), ref, rtol=1e-13, atol=1e-13)


def test_relu_score_on_positive_orthant_is_weighted_matmul():
    rng = np.random.default_rng(1)
    T, H, D, N = 4, 3, 8, 29
    q = np.abs(rng.standard_normal((T, H, D)))
    kk = np.abs(rng.standard_normal((N, D)))
    W = rng.random((T, H))
    c = _case(T, H, D, N, 3, q=q, kk=kk, W=W)
    qf, kf, wf = (c.q_bits.astype(np.float64), c.k_bits.astype(np.float64), c.W.astype(np.float64))
    # sum_h w[t,h] q[t,h,:] . k[j,:]  ==  (sum_h w[t,h] q[t,h,:]) @ K^T
    ref = np.stack([(wf[t] @ qf[t]) @ kf.T for t in range(T)])
    np.testing.assert_allclose(_all_rows(c), ref, rtol=1e-12)


def test_negated_heads_contribute_nothing():
    rng = np.random.default_rng(2)
    T, H, D, N = 3, 4, 6, 17
    q = np.abs(rng.standard_normal((T, H, D)))
    q[:, 1] *= -1.0  # head 1 always scores <= 0 against positive keys
    q[2, 3] *= -1.0  # and head 3 of query 2
    kk = np.abs(rng.standard_normal((N, D)))
    W = rng.random((T, H))
    c = _case(T, H, D, N, 3, q=q, kk=kk, W=W)
    qf, kf, wf = (c.q_bits.astype(np.float64), c.k_bits.astype(np.float64), c.W.astype(np.float64).copy())
    wf[:, 1] = 0.0
    wf[2, 3] = 0.0
    ref = np.stack([(wf[t] @ qf[t]) @ kf.T for t in range(T)])
    np.testing.assert_allclose(_all_rows(c), ref, rtol=1e-12, atol=1e-15)
    # and the weights are per query: swapping two queries' weights changes rows
    c2 = _case(T, H, D, N, 3, q=q, kk=kk, W=W[::-1].copy())
    assert not np.allclose(_all_rows(c2)[0], _all_rows(c)[0])


def test_fp8_per_key_scale_is_positively_homogeneous():
    rng = np.random.default_rng(3)
    T, H, D, N = 2, 3, 16, 21
    kk = rng.standard_normal((N, D)).astype(np.float32)
    ones = np.ones(N, np.float32)
    scales = (2.0 ** rng.integers(-3, 4, size=N)).astype(np.float32)  # exact powers of two
    base = _case(T, H, D, N, 4, kk=kk, k_dtype=synth.FP8_E4M3, k_scale=ones)
    scaled = _case(T, H, D, N, 4, kk=kk, k_dtype=synth.FP8_E4M3, k_scale=scales)
    np.testing.assert_allclose(_all_rows(scaled), _all_rows(base) * scales[None, :], rtol=1e-13)


def test_monotone_keys_select_last_valid_keys():
    # D = 1, q = 1, k_j = j/64: every score is (sum_h w) * j/64, increasing in j,
    # so the Top-k of query t is the last k keys below kv_len[t].
    T, H, N, k = 4, 2, 300, 16
    q = np.ones((T, H, 1))
    kk = (np.arange(N, dtype=np.float64) / 64.0)[:, None]
    kv_len = np.array([300, 250, 16, 5])
    c = _case(T, H, 1, N, k, q=q, kk=kk, kv_len=kv_len)
    idx, val, n = oracle.fused_topk(c)
    for t in range(T):
        L = int(kv_len[t])
        exp = list(range(L - 1, max(L - k, 0) - 1, -1))
        assert n[t] == min(k, L)
        assert list(idx[t, :n[t]]) == exp
        assert (idx[t, n[t]:] == -1).all() and np.isneginf(val[t, n[t]:]).all()


def test_all_relu_zero_rows_select_lowest_indices():
    rng = np.random.default_rng(4)
    T, H, D, N, k = 2, 3, 8, 50, 7
    q = -np.abs(rng.standard_normal((T, H, D)))
    kk = np.abs(rng.standard_normal((N, D)))
    c = _case(T, H, D, N, k, q=q, kk=kk)
    idx, val, n = oracle.fused_topk(c)
    assert (val[:, :k] == 0.0).all()
    assert (idx == np.arange(k)[None, :]).all()


def test_fused_topk_matches_selection_of_score_row():
    c = synth.gen_fused(6, 4, 16, 200, 9, q_dtype=synth.BF16, k_dtype=synth.BF16,
                        kv_len=[200, 150, 9, 3, 1, 120], seed=11)
    idx, val, n = oracle.fused_topk(c, nthreads=3)
    sidx, sval, sn = oracle.fused_topk(c, rows=[3, 0], nthreads=1)
    assert np.array_equal(sidx, idx[[3, 0]]) and np.array_equal(sval, val[[3, 0]])
    for t in range(c.T):
        row = oracle.fused_score_row(c, t)
        order = np.lexsort((np.arange(row.size), -row))[: c.k]
        assert n[t] == min(c.k, row.size)
        assert list(idx[t, :n[t]]) == list(order)
        pairs = oracle.fused_scores_at(c, np.full(n[t], t), idx[t, :n[t]])
        assert np.array_equal(pairs, val[t, :n[t]])


# -------------------------------------------------------- selection pins
def _brute_force_topk_set(x, k):
    """Enumerate every subset of size min(k, L); keep those that beat every
    outsider under (value desc, index asc).  Exactly one must survive."""
    L = len(x)
    m = min(k, L)
    winners = []
    for S in itertools.combinations(range(L), m):
        inside = set(S)
        ok = all((x[i] > x[j]) or (x[i] == x[j] and i < j)
                 for i in inside for j in range(L) if j not in inside)
        if ok:
            winners.append(inside)
    assert len(winners) == 1
    return winners[0]


def test_selection_against_subset_enumeration():
    rng = np.random.default_rng(5)
    pool = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 3.0, np.inf, -np.inf], dtype=np.float32)
    for trial in range(300):
        L = int(rng.integers(0, 9))
        k = int(rng.integers(1, 5))
        x = rng.choice(pool, size=L).astype(np.float32)
        idx, n = oracle.select(x, k)
        assert n == min(k, L)
        assert set(idx[:n].tolist()) == _brute_force_topk_set(x.tolist(), k)
        assert (idx[n:] == -1).all()


def test_selection_order_against_repeated_argmax():
    rng = np.random.default_rng(6)
    for trial in range(100):
        L = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        x = rng.integers(-3, 4, size=L).astype(np.float32)
        idx, n = oracle.select(x, k)
        taken = np.zeros(L, bool)
        for r in range(n):
            best = -1
            for j in range(L):  # first maximum among the untaken = lowest index
                if not taken[j] and (best < 0 or x[j] > x[best]):
                    best = j
            taken[best] = True
            assert idx[r] == best


@pytest.mark.parametrize("family", synth.RAGGED_FAMILIES)
def test_ragged_exactness_invariants(family):
    c = synth.gen_ragged(6, 4096, 300, lens=[4096, 3000, 300, 299, 1, 0], seed=9, family=family)
    idx, n = oracle.topk_ragged(c)
    for r in range(c.M):
        L = int(c.row_len[r])
        x = c.scores[r, :L].astype(np.float64)
        sel = idx[r, :n[r]]
        assert n[r] == min(c.k, L)
        assert len(set(sel.tolist())) == n[r]
        assert ((sel >= 0) & (sel < L)).all() and (idx[r, n[r]:] == -1).all()
        if 0 < n[r] < L:
            # Eq. (30): min over selected >= max over the rest
            mask = np.ones(L, bool)
            mask[sel] = False
            assert x[sel].min() >= x[mask].max()
            # ties at the boundary go to the lowest indices
            kth = x[sel].min()
            eq = np.flatnonzero(x == kth)
            n_above = int((x > kth).sum())
            assert set(sel[x[sel] == kth].tolist()) == set(eq[: n[r] - n_above].tolist())
        order = np.lexsort((np.arange(L), -x))[: c.k]
        assert list(sel) == list(order)


def test_ragged_ignores_padded_tail_and_signed_zero_ties():
    scores = np.full((2, 8), np.inf, np.float32)  # +inf beyond row_len must be ignored
    scores[0, :5] = [-0.0, 0.0, -0.0, -1.0, 0.0]
    scores[1, :3] = [1.0, 2.0, 3.0]
    c = synth.RaggedCase(name="z", M=2, pitch=8, k=2, scores=scores, row_len=np.array([5, 3], np.int32))
    idx, n = oracle.topk_ragged(c)
    assert list(idx[0]) == [0, 1]  # -0 == +0: lowest indices win
    assert list(idx[1]) == [2, 1]


def test_special_rows():
    L, k = 1000, 64
    idx, n = oracle.select(np.full(L, 0.5, np.float32), k)
    assert list(idx) == list(range(k))
    idx, n = oracle.select(np.arange(L, dtype=np.float32), k)
    assert list(idx) == list(range(L - 1, L - 1 - k, -1))
    idx, n = oracle.select(np.arange(10, dtype=np.float32), k)
    assert n == 10 and list(idx[:10]) == list(range(9, -1, -1)) and (idx[10:] == -1).all()
    idx, n = oracle.select(np.zeros(0, np.float32), k)
    assert n == 0 and (idx == -1).all()


# --------------------------------------------------- length clamping pins
def test_fused_lengths_are_clamped_to_zero_and_n():
    """L_t = min(max(kv_len[t], 0), N): a length past N selects like N, a
    negative one like 0 (the operator contract of the Sample-Guided Exact
    Top-K paper, Sec. 2.1: only valid entries are read)."""
    c = synth.gen_fused(4, 3, 16, 120, 10, q_dtype=synth.BF16, k_dtype=synth.BF16,
                        kv_len=[120, 120 + 77, -4, 0], seed=21)
    c.q_bits[1], c.W[1] = c.q_bits[0], c.W[0]  # rows 0 and 1 differ only in kv_len
    idx, val, n = oracle.fused_topk(c)
    assert list(n) == [10, 10, 0, 0]
    assert np.array_equal(idx[0], idx[1]) and np.array_equal(val[0], val[1])
    assert (idx[2:] == -1).all() and np.isneginf(val[2:]).all()
    assert oracle.fused_score_row(c, 1).size == 120 and oracle.fused_score_row(c, 2).size == 0
    assert oracle.valid_len(c, 1) == 120 and oracle.valid_len(c, 2) == 0
    with pytest.raises(RuntimeError):
        oracle.fused_scores_at(c, [0], [120])


def test_ragged_lengths_are_clamped_to_zero_and_pitch():
    c = synth.gen_ragged(3, 64, 8, lens=[64, 64, 64], seed=3)
    c.row_len = np.array([64, 64 + 5, -2], np.int32)
    idx, n = oracle.topk_ragged(c)
    assert list(n) == [8, 8, 0]
    ref, _ = oracle.select(c.scores[1, :64], 8)
    assert list(idx[1]) == list(ref) and (idx[2] == -1).all()


# ------------------------------------------------- e4m3fn encoder pins
def test_encode_e4m3_every_fp32_pattern_against_torch():
    """The encoder (written from the OCP E4M3 value set, round to nearest,
    ties to even) against torch's float8_e4m3fn cast on all 2^32 fp32 bit
    patterns; NaN codes are compared as NaN."""
    import torch
    chunk = 1 << 26
    for c in range((1 << 32) // chunk):
        bits = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint32)
        x = bits.view(np.float32)
        ours = oracle.encode_e4m3(x)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        both_nan = ((ours & 0x7F) == 0x7F) & ((ref & 0x7F) == 0x7F)
        bad = (ours != ref) & ~both_nan
        assert not bad.any(), f"fp32 0x{int(bits[np.argmax(bad)]):08x}: {ours[bad][:4]} vs {ref[bad][:4]}"


def test_encode_e4m3_landmarks():
    # ties to even at 2^-10 (half the smallest subnormal) and at 464 (between
    # 448 and the NaN code); 1.0625 is halfway between 1 and 1.125
    x = np.array([2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 448, 464, 464.5, -0.0], np.float32)
    assert list(oracle.encode_e4m3(x)) == [0x00, 0x02, 0x38, 0x3A, 0x7E, 0x7E, 0x7F, 0x80]


# ---------------------------------------------------- FP8 scoring pins
FP8_SCORE = 2


def test_fp8_scoring_worked_example():
    """Quantized-query scoring worked by hand (LiteTopK Sec. 2.1: FP8 indexer).

    Head 0, q = [1, 0.5, -0.30078125, 0.10009765625] (bf16 values): a = 1,
    448 / a = 448, products 448, 224, -134.75, 44.84375.  In e4m3fn the
    spacing is 32 on [256, 512), 16 on [128, 256), 4 on [32, 64): codes
    448, 224, -128 (134.75 / 16 = 8.42 -> 8), 44 (44.84 / 4 = 11.2 -> 11);
    scale s0 = fp32(1 / 448).
    Head 1, q = [-2, 0.75, 3, 0]: a = 3, 448 / 3 = 149.333336 (fp32);
    products -298.67, 112.0000019 (-> fp32 112), 448.0000076 (-> fp32 448), 0:
    codes -288 (298.67 / 32 = 9.33 -> 9), 112, 448, 0; s1 = fp32(3 / 448).
    FP8 keys (scale 1): k0 = e0, k1 = e2, k2 = [1, 1, 1, 1]; W = [0.5, 0.25].
    Head dots: k0 -> 448, -288; k1 -> -128, 448; k2 -> 588, 272."""
    q = np.array([[[1.0, 0.5, -0.30078125, 0.10009765625], [-2.0, 0.75, 3.0, 0.0]]], np.float32)
    kk = np.array([[1, 0, 0, 0], [0, 0, 1, 0], [1, 1, 1, 1]], np.float32)
    c = _case(1, 2, 4, 3, 3, q=q, kk=kk, W=np.array([[0.5, 0.25]]), q_dtype=synth.BF16,
              k_dtype=synth.FP8_E4M3, k_scale=np.ones(3, np.float32))
    s0 = float(np.float32(1.0) / np.float32(448.0))
    s1 = float(np.float32(3.0) / np.float32(448.0))
    c.flags = FP8_SCORE
    exp = np.array([0.5 * s0 * 448, 0.25 * s1 * 448, 0.5 * s0 * 588 + 0.25 * s1 * 272])
    np.testing.assert_array_equal(oracle.fused_score_row(c, 0), exp)
    idx, val, n = oracle.fused_topk(c)
    assert list(idx[0]) == [2, 1, 0] and np.array_equal(val[0], exp[[2, 1, 0]])
    # without the flag: the plain score of the unquantized queries
    c.flags = 0
    plain = np.array([0.5, 0.25 * 3.0, 0.5 * (1 + 0.5 - 0.30078125 + 0.10009765625) + 0.25 * 1.75])
    np.testing.assert_allclose(oracle.fused_score_row(c, 0), plain, rtol=1e-15)


def test_fp8_scoring_is_identity_on_representable_rows():
    """Rows whose values are e4m3fn values times 2^-6 with a largest
    magnitude of 7 (= 448 * 2^-6): 448 / 7 = 64 and 7 / 448 = 2^-6 exactly,
    every product is an e4m3fn value, so the quantized score equals the plain
    score exactly."""
    rng = np.random.default_rng(31)
    T, H, D, N = 3, 5, 32, 40
    codes = oracle.decode(rng.integers(0, 256, size=(T, H, D)).astype(np.uint8), synth.FP8_E4M3)
    codes = np.where(np.isnan(codes), 0.0, codes)
    codes[..., 0] = 448.0 * np.sign(rng.standard_normal((T, H)))
    q = (codes * 2.0 ** -6).astype(np.float32)
    kk = rng.standard_normal((N, D)).astype(np.float32)
    scale = (2.0 ** rng.integers(-3, 3, size=N)).astype(np.float32)
    c = _case(T, H, D, N, 6, q=q, kk=kk, q_dtype=synth.BF16, k_dtype=synth.FP8_E4M3, k_scale=scale)
    plain = _all_rows(c)
    c.flags = FP8_SCORE
    np.testing.assert_array_equal(_all_rows(c), plain)


def test_fp8_scoring_within_quantization_bound():
    """Each quantized element moves by at most 2^-4 of itself (three fraction
    bits, round to nearest) or, below the normal range, by 2^-10 of the row's
    scale; ReLU is 1-Lipschitz, so |I8 - I| <= sum_h w_h sum_d
    (2^-4 |q_hd| + 2^-10 s_h) |k_d|.  The bound is met and not vacuous: the
    error is a small fraction of the score."""
    c = synth.gen_fused(4, 8, 64, 300, 5, q_dtype=synth.BF16, k_dtype=synth.FP8_E4M3, seed=33)
    exact = _all_rows(c)
    c.flags = FP8_SCORE
    quant = _all_rows(c)
    q = oracle.decode(c.q_bits, synth.BF16).reshape(c.T, c.H, c.D)
    k = oracle.decode(c.k_bits, synth.FP8_E4M3).reshape(c.N, c.D) * c.k_scale[:, None]
    for t in range(c.T):
        s = np.abs(q[t]).max(axis=1) / 448.0
        per_head = 2.0 ** -4 * (np.abs(q[t]) @ np.abs(k).T) + 2.0 ** -10 * s[:, None] * np.abs(k).sum(1)[None]
        bound = (c.W[t].astype(np.float64)[:, None] * per_head).sum(0)
        err = np.abs(quant[t] - exact[t])
        assert (err <= bound * (1 + 1e-12)).all()
        assert err.max() > 0 and np.median(err / np.maximum(np.abs(exact[t]), 1e-12)) < 0.05


# ---- history sample (LiteTopK Sec. 3.2 "Sampling": the k' keys most frequent
# in the previous chunk's Top-k lists)

def test_prior_worked_example():
    """Counts by hand: key 1 three times, key 3 twice, keys 4 and 5 once,
    keys 0 and 2 never; -1 padding and the out-of-range 9 count for nothing.
    Equal counts go to the lower index, and slots past N hold -1."""
    prev = np.array([[3, 1, -1], [1, 4, 3], [5, 1, 9]], dtype=np.int32)
    assert oracle.prior_from_topk(prev, 6, 4).tolist() == [1, 3, 4, 5]
    assert oracle.prior_from_topk(prev, 6, 5).tolist() == [1, 3, 4, 5, 0]
    assert oracle.prior_from_topk(prev, 6, 8).tolist() == [1, 3, 4, 5, 0, 2, -1, -1]
    # a key range that ends below the listed keys drops them
    assert oracle.prior_from_topk(prev, 4, 4).tolist() == [1, 3, 0, 2]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prior_against_counter_brute_force(seed):
    import collections
    rng = np.random.default_rng(seed)
    N = int(rng.integers(5, 200))
    T, k = int(rng.integers(1, 12)), int(rng.integers(1, 20))
    prev = rng.integers(-3, N + 3, size=(T, k)).astype(np.int32)
    cnt = collections.Counter(int(j) for j in prev.ravel() if 0 <= j < N)
    order = sorted(range(N), key=lambda j: (-cnt[j], j))
    for kp in (1, 3, N // 2 + 1, N, N + 5):
        want = order[:min(kp, N)] + [-1] * max(0, kp - N)
        assert oracle.prior_from_topk(prev, N, kp).tolist() == want


def test_prior_of_disjoint_lists_is_most_repeated_first():
    """Each key of block b appears in b + 1 of the lists, so the blocks come
    out in decreasing repetition, each in index order."""
    N, k = 40, 8
    rows = []
    for b in range(4):  # keys 8b .. 8b+7 appear in b+1 rows
        rows += [np.arange(8 * b, 8 * b + 8, dtype=np.int32)] * (b + 1)
    prev = np.stack(rows)
    got = oracle.prior_from_topk(prev, N, 32).tolist()
    assert got == list(range(24, 32)) + list(range(16, 24)) + list(range(8, 16)) + list(range(0, 8))
