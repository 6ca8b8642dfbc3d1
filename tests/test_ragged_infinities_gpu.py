"""Rows where infinities decide the selection, against the oracle (bit-exact
sets on both selector mappings).

±inf are ordered like any other value and equal values go to the lower
index (SGTK Sec. 2.1 "Operator contract"; ties as in the project's
contract).  These rows stress the parts that look at the value range: a
row with more than k entries at +inf (the view's range is infinite, and the
whole Top-k is the lowest-index +inf entries), a row whose finite values
number fewer than k among -inf (the -inf entries are selected, lowest
indices first), a row of -inf only, and ±inf among ordinary values."""
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


def _rows(M, pitch, k, seed):
    rng = np.random.default_rng(seed)
    x = np.full((M, pitch), -np.inf, dtype=np.float32)
    lens = rng.integers(pitch // 2, pitch + 1, size=M).astype(np.int32)
    for r in range(M):
        L = int(lens[r])
        kind = r % 4
        row = rng.standard_normal(L).astype(np.float32)
        if kind == 0:    # more than k entries at +inf
            row[rng.choice(L, size=min(L, 2 * k), replace=False)] = np.inf
        elif kind == 1:  # fewer than k finite values, the rest -inf
            row[:] = -np.inf
            row[rng.choice(L, size=k // 3, replace=False)] = rng.standard_normal(k // 3).astype(np.float32)
        elif kind == 2:  # -inf only
            row[:] = -np.inf
        else:            # a few of each among ordinary values, and a huge finite value
            row[rng.choice(L, size=5, replace=False)] = np.inf
            row[rng.choice(L, size=5, replace=False)] = -np.inf
            row[rng.integers(0, L)] = np.float32(3e38)
        x[r, :L] = row
    return synth.RaggedCase(name="ragged_infinities", M=M, pitch=pitch, k=k, scores=x, row_len=lens)


@pytest.mark.parametrize("route", [1, 2, 3])       # segmented, row-local, row-local direct-exact
@pytest.mark.parametrize("M,pitch,k", [(8, 40_000, 512), (16, 9_000, 2048)])
def test_infinities_select_exactly(itk, route, M, pitch, k):
    itk.set_plan_opts(ragged_route=route)
    case = _rows(M, pitch, k, seed=M + k)
    out = itk.topk_ragged(torch.from_numpy(case.scores).cuda(), torch.from_numpy(case.row_len).cuda(), k)
    torch.cuda.synchronize()
    check_ragged_exact(case, out.cpu().numpy())
