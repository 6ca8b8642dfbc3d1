"""Large k against the oracle: k above the on-chip stash of the selection
(7680 items) and k close to or above the row length.

Rows whose candidates exceed the stash are refined straight from the
candidate buffer (or the row) in global memory, with the same radix digits.
The shapes with k above the stash take that route on every mapping they use;
the other tests reach it only through forced overflows.  Bit-exact: the standalone selector on fp32 rows,
and the fused call on the integer family, whose scores are exact in fp32
(SGTK Sec. 2.1 "Operator contract"; LiteTopK Sec. 2.1 Eq. (1))."""
import numpy as np
import pytest
import torch

import synth
from parity import check_fused_exact, check_ragged_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset(itk):
    itk.reset_plan_opts()
    yield
    itk.reset_plan_opts()


@pytest.mark.parametrize("M,pitch,k,family", [
    (6, 200_000, 16_384, "config2"),     # k above the stash, rows 8x longer
    (4, 40_000, 30_000, "ties_at_k"),    # k close to the row length, ties at the boundary
    (5, 20_000, 65_536, "few_values"),   # k above every row length: whole rows
    (600, 12_000, 9_000, "config2"),     # many rows (segmented: k too large for the row-local mapping)
])
def test_ragged_large_k(itk, M, pitch, k, family):
    rng = np.random.default_rng(M + k)
    lens = rng.integers(pitch // 2, pitch + 1, size=M).astype(np.int32)
    lens[0] = pitch
    case = synth.gen_ragged(M, pitch, k, lens=lens, seed=k, family=family)
    x = torch.from_numpy(case.scores).cuda()
    rl = torch.from_numpy(case.row_len).cuda()
    out = itk.topk_ragged(x, rl, k)
    torch.cuda.synchronize()
    check_ragged_exact(case, out.cpu().numpy())


@pytest.mark.parametrize("T,H,D,N,k,kdt", [
    (8, 16, 64, 40_000, 10_000, synth.BF16),       # head rows, k above the stash
    (2, 64, 128, 30_000, 12_000, synth.FP8_E4M3),  # two queries (one key range per wave), FP8 keys
    (40, 1, 128, 20_000, 9_000, synth.F16),        # single head
    (8, 8, 64, 5_000, 6_000, synth.BF16),          # k above N: every valid key
])
def test_fused_large_k_bit_exact(itk, T, H, D, N, k, kdt):
    qdt = synth.F16 if kdt == synth.F16 else synth.BF16
    rng = np.random.default_rng(k)
    kv = rng.integers(N // 2, N + 1, size=T).astype(np.int32)
    kv[0] = N
    case = synth.gen_fused_exact(T, H, D, N, k, q_dtype=qdt, k_dtype=kdt, kv_len=kv, seed=k,
                                 no_relu=(H == 1))
    Q, K, S, W, kvt = itk.fused_tensors(case)
    idx, sc = itk.indexer_topk_fused(Q, K, W, kvt, k, k_scale=S, flags=case.flags)
    torch.cuda.synchronize()
    check_fused_exact(case, range(T), idx.cpu().numpy(), sc.cpu().numpy())
