"""topk_ragged_noalloc (static per-GPU scratch, no workspace) against
topk_ragged on the same inputs, through the C ABI: two calls in a row, the
second smaller, each equal to the workspace call's result (and to the
oracle's); no device memory is taken by a call after the first; shapes
beyond the static scratch are rejected with nothing enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from parity import check_ragged_exact

pytestmark = pytest.mark.gpu


def _both(itk, case):
    x = torch.from_numpy(case.scores).cuda()
    rl = torch.from_numpy(case.row_len).cuda()
    ref = itk.topk_ragged(x, rl, case.k)
    out = torch.full((case.M, case.k), -7, dtype=torch.int32, device="cuda")
    itk.topk_ragged_noalloc(x, rl, case.k, out)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


def _free_bytes():
    free, _total = torch.cuda.mem_get_info()
    return free


def test_noalloc_matches_workspace_call_twice(itk):
    # rows longer than 2^18 scores take the segmented route, whose per-segment
    # slices live in the static scratch: 8 rows of 2^20, then a smaller call
    big = synth.gen_ragged(8, 1 << 20, 2048, lens=[1 << 20, (1 << 20) - 77, 500000, 2048, 2047, 0, 300001, 1 << 20],
                           seed=41)
    small = synth.gen_ragged(3, 300000, 700, lens=[300000, 299999, 65537], seed=42, family="ties_at_k")
    assert itk.topk_ragged_workspace_size(big.M, big.pitch, big.k) > itk.topk_ragged_workspace_size(
        small.M, small.pitch, small.k)
    for case in (big, small):
        ref, got = _both(itk, case)
        assert np.array_equal(np.sort(ref, axis=1), np.sort(got, axis=1))
        check_ragged_exact(case, got)
    # shorter rows (the row-local route, no scratch), two calls in a row
    for case in (synth.ragged_config(),
                 synth.gen_ragged(9, 20000, 100, lens=[20000, 19999, 100, 99, 1, 0, 20000 + 5, -3, 7777], seed=4)):
        ref, got = _both(itk, case)
        assert np.array_equal(np.sort(ref, axis=1), np.sort(got, axis=1))
        check_ragged_exact(case, got)
    # the call takes no device memory: free memory is unchanged over calls
    x = torch.from_numpy(small.scores).cuda()
    rl = torch.from_numpy(small.row_len).cuda()
    out = torch.empty((small.M, small.k), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    free1 = _free_bytes()
    for _ in range(3):
        itk.topk_ragged_noalloc(x, rl, small.k, out)
    torch.cuda.synchronize()
    assert _free_bytes() == free1
    check_ragged_exact(small, out.cpu().numpy())


def test_noalloc_rejects_shapes_beyond_the_scratch(itk):
    lib = itk.lib()
    need = lib.topk_ragged_workspace_size(64, 1 << 20, 2048)  # 64 rows of 2^20 scores: segmented route
    assert need > itk.RAGGED_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, 16), dtype=torch.float32, device="cuda")
    st = lib.topk_ragged_noalloc(ctypes.c_void_p(x.data_ptr()), 1 << 20, ctypes.c_void_p(x.data_ptr()), 64, 2048,
                                 ctypes.c_void_p(x.data_ptr()), None)
    assert st == 5 and lib.itk_status_string(5).startswith(b"shape needs more")
