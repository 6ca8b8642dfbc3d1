"""Empty problems through the C ABI: no rows, k == 0, and no keys (N == 0 for
the fused call, row pitch 0 for the standalone selector).

Both operator contracts (SGTK Sec. 2.1 "Operator contract"; LiteTopK
Sec. 2.1 Eq. (1)) return the min(k, L) best indices of each row, so a row
with no valid key gets only the padding (-1, and -inf scores), and a call
without rows or with k == 0 has nothing to return.  The padded outputs are
compared with the oracle's on the same shapes; the calls with nothing to
return must succeed and leave their (empty) outputs alone."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("k_dtype", [synth.BF16, synth.FP8_E4M3])
def test_fused_without_keys_pads_every_row(itk, k_dtype):
    case = synth.gen_fused(5, 8, 64, 0, 16, k_dtype=k_dtype, seed=1)  # N = 0
    want_i, want_v, want_n = oracle.fused_topk(case)
    assert (want_n == 0).all()
    Q, K, S, W, kv = itk.fused_tensors(case)
    oi = torch.full((5, 16), 7, dtype=torch.int32, device="cuda")
    os_ = torch.full((5, 16), 3.0, dtype=torch.float32, device="cuda")
    itk.indexer_topk_fused(Q, K, W, kv, 16, k_scale=S, out_idx=oi, out_score=os_)
    torch.cuda.synchronize()
    assert np.array_equal(oi.cpu().numpy(), want_i)
    assert np.array_equal(os_.cpu().numpy().astype(np.float64), want_v)
    # the history-sample call takes the same path
    oi.fill_(7)
    prior = torch.tensor([0, 3, 9], dtype=torch.int32, device="cuda")
    itk.indexer_topk_fused_prior(Q, K, W, kv, 16, prior, k_scale=S, out_idx=oi, out_score=os_)
    torch.cuda.synchronize()
    assert np.array_equal(oi.cpu().numpy(), want_i)


def test_fused_without_queries_or_k(itk):
    g = torch.Generator(device="cpu").manual_seed(3)
    K = torch.randn(100, 64, generator=g).to(torch.bfloat16).cuda()
    Q0 = torch.empty((0, 8, 64), dtype=torch.bfloat16, device="cuda")
    W0 = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    kv0 = torch.empty(0, dtype=torch.int32, device="cuda")
    oi, os_ = itk.indexer_topk_fused(Q0, K, W0, kv0, 16)
    assert oi.shape == (0, 16) and os_.shape == (0, 16)
    # k == 0: nothing to return for any query
    Q = torch.randn(4, 8, 64, generator=g).to(torch.bfloat16).cuda()
    W = torch.rand(4, 8, generator=g).cuda()
    kv = torch.full((4,), 100, dtype=torch.int32, device="cuda")
    oi, os_ = itk.indexer_topk_fused(Q, K, W, kv, 0)
    torch.cuda.synchronize()
    assert oi.shape == (4, 0) and os_.shape == (4, 0)
    # the same shape with k = 8 still runs (the empty calls left no state behind)
    case_i, _ = itk.indexer_topk_fused(Q, K, W, kv, 8)
    torch.cuda.synchronize()
    assert ((case_i.cpu().numpy() >= 0) & (case_i.cpu().numpy() < 100)).all()


@pytest.mark.parametrize("noalloc", [False, True])
def test_ragged_rows_of_pitch_zero_are_padding(itk, noalloc):
    case = synth.gen_ragged(4, 0, 8, lens=np.array([0, 3, 0, 5]), seed=1)
    want, want_n = oracle.topk_ragged(case)
    assert (want_n == 0).all()
    out = torch.full((4, 8), 7, dtype=torch.int32, device="cuda")
    lib = itk.lib()
    if noalloc:
        st = lib.topk_ragged_noalloc(None, 0, None, 4, 8, ctypes.c_void_p(out.data_ptr()), _stream())
    else:
        st = lib.topk_ragged(None, 0, None, 4, 8, ctypes.c_void_p(out.data_ptr()), None, 0, _stream())
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want)


def test_ragged_without_rows_or_k(itk):
    scores = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    row_len = torch.empty(0, dtype=torch.int32, device="cuda")
    assert itk.topk_ragged(scores, row_len, 8).shape == (0, 8)
    scores = torch.randn(4, 128, device="cuda")
    row_len = torch.full((4,), 128, dtype=torch.int32, device="cuda")
    assert itk.topk_ragged(scores, row_len, 0).shape == (4, 0)
    out = torch.empty((4, 0), dtype=torch.int32, device="cuda")
    assert itk.topk_ragged_noalloc(scores, row_len, 0, out).shape == (4, 0)
    torch.cuda.synchronize()
