"""History-guided sample (LiteTopK Sec. 3.2 "Sampling") on the GPU.

indexer_prior_from_topk against the oracle's definition (bit-exact sets: the
order by (count descending, index ascending) is unique), and
indexer_topk_fused_prior against the oracle: the prior only places the
initial gate, so the result is the exact Top-k whatever the list holds.
Bit-exact on the integer family (scores exact in fp32) with good, random,
duplicated, out-of-range, empty-for-some-rows and adversarial lists; within
the fp32 bar on consecutive prefill chunks, where the list comes from the
previous chunk's own output and the count knob shows the tighter gate."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_fused_exact, check_fused_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset(itk):
    itk.reset_plan_opts()
    yield
    itk.reset_plan_opts()


# N = 2^20 spans 32 key ranges of the counting step, so its entries are
# counted one global atomic each; the others count through LDS per range.
@pytest.mark.parametrize("T,k,N,kp,seed", [(7, 20, 300, 50, 1), (64, 256, 4096, 768, 2), (3, 5, 40, 64, 3),
                                           (0, 8, 100, 10, 4), (300, 2048, 133120, 6144, 5),
                                           (64, 512, 1 << 20, 1536, 6)])
def test_prior_from_topk_matches_oracle(itk, T, k, N, kp, seed):
    rng = np.random.default_rng(seed)
    # skewed key popularity, -1 padding and entries outside [0, N)
    pop = rng.zipf(1.3, size=(T, k)) % (N + 7) - 3
    prev = pop.astype(np.int32)
    want = oracle.prior_from_topk(prev.reshape(T, k), N, kp)
    got = itk.prior_from_topk(torch.from_numpy(prev.reshape(T, k)).cuda(), N, kp)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    n = min(kp, N)
    assert (g[n:] == -1).all()
    # the list comes out in ascending index order
    assert g[:n].tolist() == sorted(want[:n].tolist())


@pytest.mark.parametrize("kp", [3, 8, 20])
def test_prior_counts_above_4096(itk, kp):
    """Counts in the second bin of the first histogram level and beyond
    (5000 and 9000 repeats), ties at the boundary count, and padding."""
    rng = np.random.default_rng(kp)
    T, k, N = 9000, 8, 3000
    prev = rng.integers(0, N, size=(T, k)).astype(np.int32)
    prev[:, 0] = 17                       # 9000 occurrences
    prev[:5000, 1] = 2999                 # 5000 and more
    prev[:5000, 2] = 5                    # a tie with 2999 at 5000 (before the random hits)
    prev[5000:, 1] = 1000
    want = oracle.prior_from_topk(prev, N, kp)
    got = itk.prior_from_topk(torch.from_numpy(prev).cuda(), N, kp).cpu().numpy()
    assert got.tolist() == sorted(want.tolist())


def _fused(itk, case, prior, count=False, routes=False):
    Q, K, S, W, kv = itk.fused_tensors(case)
    pr = torch.from_numpy(np.ascontiguousarray(prior, dtype=np.int32)).cuda()
    cnt = torch.full((case.T,), -1, dtype=torch.int32, device="cuda")
    rb = torch.zeros(case.T, dtype=torch.int32, device="cuda")
    if count:
        itk.set_count_buffer(cnt)
    if routes:
        itk.set_route_buffer(rb)
    try:
        idx, sc = itk.indexer_topk_fused_prior(Q, K, W, kv, case.k, pr, k_scale=S, flags=case.flags)
        torch.cuda.synchronize()
    finally:
        itk.set_count_buffer(None)
        itk.set_route_buffer(None)
    return idx.cpu().numpy(), sc.cpu().numpy(), cnt.cpu().numpy(), rb.cpu().numpy()


T, N, K = 19, 9000, 300
KV = np.array([N, N - 1, 8000, K + 1, K, K - 1, 1, 0, 64, 65, 4500, N + 321, -9] +
              [N - 37 * i for i in range(6)], dtype=np.int32)


def _priors(case, rng):
    """Lists of every kind; the good one is the oracle Top-3k of row 0."""
    o_idx, _, o_n = oracle.fused_topk(case, rows=[0])
    good = oracle.fused_topk(synth.FusedCase(**{**case.__dict__, "k": 3 * case.k}), rows=[0])[0][0]
    good = good[good >= 0]
    worst = np.argsort(oracle.fused_score_row(case, 0), kind="stable")[:3 * case.k]
    return {
        "good": good,
        "random": rng.choice(case.N, size=900, replace=False),
        "duplicated": np.repeat(good[:100], 9),
        "out_of_range": np.concatenate([good[:600], [-1, -5, case.N, case.N + 10, 2 ** 31 - 1] * 20]),
        "short_rows_only": np.arange(0, 400),
        "worst_keys": worst,
        "fewer_than_k": good[:K - 1],
        "one_tile": good[:64],
    }


@pytest.mark.parametrize("qt,kt,H,D,fp8", [(synth.BF16, synth.BF16, 64, 128, False),
                                           (synth.F16, synth.FP8_E4M3, 20, 128, False),
                                           (synth.F32, synth.F32, 40, 64, False),
                                           (synth.BF16, synth.FP8_E4M3, 64, 128, True)])
def test_fused_prior_bit_exact(itk, qt, kt, H, D, fp8):
    case = synth.gen_fused_exact(T, H, D, N, K, q_dtype=qt, k_dtype=kt, kv_len=KV, fp8_score=fp8,
                                 seed=H * 13 + D + fp8)
    rng = np.random.default_rng(H)
    for name, prior in _priors(case, rng).items():
        idx, sc, cnt, rt = _fused(itk, case, prior, count=True, routes=True)
        print(name, "routes", np.bincount(rt, minlength=6).tolist())
        check_fused_exact(case, range(T), idx, sc)


@pytest.mark.parametrize("T_", [1, 2, 9])
def test_fused_prior_few_queries(itk, T_):
    """The few-query scan (one key range per wave) and a grid with fewer
    query groups than sample splits."""
    case = synth.gen_fused_exact(T_, 64, 128, 50000, 512, kv_len=np.full(T_, 50000 - 3), seed=T_)
    prior = np.random.default_rng(T_).choice(50000, size=1536, replace=False)
    idx, sc, _, _ = _fused(itk, case, prior)
    check_fused_exact(case, range(T_), idx, sc)


@pytest.mark.parametrize("knob", [dict(force_route=1), dict(capacity=K, rho=50.0), dict(splits=8)])
def test_fused_prior_under_other_plans(itk, knob):
    case = synth.gen_fused_exact(T, 64, 128, N, K, kv_len=KV, seed=99)
    prior = _priors(case, np.random.default_rng(0))["good"]
    itk.set_plan_opts(**knob)
    idx, sc, _, _ = _fused(itk, case, prior)
    check_fused_exact(case, range(T), idx, sc)


def test_consecutive_prefill_chunks(itk):
    """The previous chunk's output, through indexer_prior_from_topk, gates the
    next chunk: exact results, no recovered row, and fewer candidates per row
    than the strided view admits."""
    prev, cur = synth.prefill_chunk_pair(64, 64, 128, 16384, 512, seed=3)
    Qp, Kp_, Sp, Wp, kvp = itk.fused_tensors(prev)
    pidx, _ = itk.indexer_topk_fused(Qp, Kp_, Wp, kvp, prev.k, k_scale=Sp)
    prior = itk.prior_from_topk(pidx, prev.N, 3 * prev.k)
    torch.cuda.synchronize()
    # the prior is the oracle's definition applied to the kernel's own lists
    want = oracle.prior_from_topk(pidx.cpu().numpy(), prev.N, 3 * prev.k)
    assert prior.cpu().numpy().tolist() == sorted(want.tolist())
    idx, sc, cnt, rt = _fused(itk, cur, prior.cpu().numpy(), count=True, routes=True)
    check_fused_rows(cur, range(cur.T), idx, sc)
    assert set(np.unique(rt).tolist()) <= {1}, np.bincount(rt).tolist()
    Q, K_, S, W, kv = itk.fused_tensors(cur)
    c0 = torch.full((cur.T,), -1, dtype=torch.int32, device="cuda")
    itk.set_count_buffer(c0)
    try:
        itk.indexer_topk_fused(Q, K_, W, kv, cur.k, k_scale=S)
        torch.cuda.synchronize()
    finally:
        itk.set_count_buffer(None)
    c0 = c0.cpu().numpy()
    print("admitted per row: history sample median", np.median(cnt), "max", cnt.max(),
          "; strided view median", np.median(c0), "max", c0.max())
    assert (cnt >= cur.k).all()
    assert np.median(cnt) < np.median(c0)
