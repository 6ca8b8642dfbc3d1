"""Row-local direct-exact steps of the standalone selector: rows whose valid
entries fit the on-chip stash are refined whole, with no view (SGTK Sec. 5.5,
the row-local exact mapping; exactness as in Sec. 6.1 Eq. (30)).

Bit-exact against the oracle under the default mapping (a pitch that fits the
stash takes the row-local mapping at any row count, and rows up to
rho1 k + 3072 take the direct steps), under route 3 (every row that fits the
stash direct), with a capacity below the row lengths, and with the forced
routes.  The route codes show which rows took the direct steps: they admit
every entry (code 4) where the sampled steps would have certified a sample
(code 1)."""
import math

import numpy as np
import pytest
import torch

import synth
from parity import check_ragged_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset(itk):
    itk.reset_plan_opts()
    yield
    itk.reset_plan_opts()


def _run(itk, case):
    x = torch.from_numpy(case.scores).cuda()
    rl = torch.from_numpy(case.row_len).cuda()
    rb = torch.zeros(case.M, dtype=torch.int32, device="cuda")
    itk.set_route_buffer(rb)
    try:
        out = itk.topk_ragged(x, rl, case.k)
        torch.cuda.synchronize()
    finally:
        itk.set_route_buffer(None)
    return out.cpu().numpy(), rb.cpu().numpy()


def _direct_max(k, stash=7680, s=64):
    """The default mapping's direct limit: rho1 k + 3072, rho1 = 7/6 max(1.5, 32 s / k)."""
    rho1 = max(1.5, 32.0 * s / k) * 7.0 / 6.0
    return min(stash, math.ceil(rho1 * k) + 3072)


@pytest.mark.parametrize("M,pitch,k,family", [
    (1, 7680, 2048, "config2"),
    (8, 4096, 64, "ties_at_k"),
    (64, 7679, 256, "few_values"),      # pitch not a multiple of 4: scalar loads
    (600, 2048, 100, "all_equal"),
    (4096, 4096, 256, "gaussian"),
    (300, 7680, 8000, "descending"),    # k above every row length
    (5, 7680, 1, "signed_zero"),
    (700, 6000, 33, "outlier"),
])
def test_short_rows_default_mapping(itk, M, pitch, k, family):
    rng = np.random.default_rng(M + pitch + k)
    lens = rng.integers(0, pitch + 1, size=M).astype(np.int32)
    lens[0] = pitch
    case = synth.gen_ragged(M, pitch, k, lens=lens, seed=M * 7 + k, family=family)
    out, routes = _run(itk, case)
    check_ragged_exact(case, out)
    L = np.clip(case.row_len, 0, pitch)
    dmax = _direct_max(k)
    direct = L <= dmax - 2
    assert (routes[direct] == 4).all(), np.unique(routes[direct])
    assert (routes[L >= dmax + 2] != 4).all()


@pytest.mark.parametrize("capacity", [0, 1000])
def test_route3_every_row_that_fits(itk, capacity):
    """Route 3 takes the direct steps for every row of at most the stash (or
    `capacity`) entries; longer rows take the sampled steps in the same
    launch."""
    rng = np.random.default_rng(capacity + 1)
    lens = rng.integers(0, 20000, size=96).astype(np.int32)
    case = synth.gen_ragged(96, 20000, 512, lens=lens, seed=capacity + 5, family="config2")
    itk.set_plan_opts(ragged_route=3, capacity=capacity)
    out, routes = _run(itk, case)
    check_ragged_exact(case, out)
    cap = capacity or 7680
    assert (routes[case.row_len <= cap] == 4).all()
    assert (routes[case.row_len > cap] != 4).all()


def test_direct_sampled_and_segments_agree(itk):
    case = synth.gen_ragged(64, 4096, 300, lens=np.random.default_rng(3).integers(300, 4097, 64).astype(np.int32),
                            seed=31, family="ties_at_k")
    outs = []
    for route in (0, 1, 2, 3):
        itk.set_plan_opts(ragged_route=route)
        out, _ = _run(itk, case)
        check_ragged_exact(case, out)
        outs.append(np.sort(out, axis=1))
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


@pytest.mark.parametrize("force", [1, 2])
def test_forced_routes_on_direct_rows(itk, force):
    """Route 3 puts these rows on the direct steps.  force_route 1 still sends
    every row through the exact route; the band pass (force_route 2) needs a
    view, so rows on the direct steps ignore it."""
    case = synth.gen_ragged(16, 6000, 700, lens=np.full(16, 6000, np.int32), seed=12, family="few_values")
    itk.set_plan_opts(force_route=force, ragged_route=3)
    out, routes = _run(itk, case)
    check_ragged_exact(case, out)
    assert (routes == (3 if force == 1 else 4)).all(), routes
