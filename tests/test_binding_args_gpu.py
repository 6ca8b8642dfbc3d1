"""Tensor checks of the binding on device tensors: each malformed argument is
rejected by name before the C ABI is called, and the well-formed call right
after runs (so nothing was enqueued by the rejected ones)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _fused_args():
    g = torch.Generator().manual_seed(1)
    Q = torch.randn(4, 8, 64, generator=g).to(torch.bfloat16).cuda()
    K = torch.randn(500, 64, generator=g).to(torch.bfloat16).cuda()
    W = torch.rand(4, 8, generator=g).cuda()
    kv = torch.full((4,), 500, dtype=torch.int32, device="cuda")
    return Q, K, W, kv


def test_fused_arguments_are_checked(itk):
    Q, K, W, kv = _fused_args()
    bad = [
        (dict(Q=Q.transpose(1, 2).contiguous().transpose(1, 2)), ValueError, "Q must be contiguous"),
        (dict(Q=Q.view(torch.int16)), TypeError, "Q must be"),
        (dict(K=K[:, :32]), ValueError, "K must be"),
        (dict(K=K.t().contiguous().t()), ValueError, "K must be contiguous"),
        (dict(W=W.half()), TypeError, "W must be torch.float32"),
        (dict(W=W[:, :4]), ValueError, "W must have shape"),
        (dict(kv=kv.long()), TypeError, "kv_len must be torch.int32"),
        (dict(kv=kv[:3]), ValueError, "kv_len must have shape"),
    ]
    for change, exc, msg in bad:
        a = dict(Q=Q, K=K, W=W, kv=kv)
        a.update(change)
        with pytest.raises(exc, match=msg):
            itk.indexer_topk_fused(a["Q"], a["K"], a["W"], a["kv"], 16)
    with pytest.raises(ValueError, match="out_idx must have shape"):
        itk.indexer_topk_fused(Q, K, W, kv, 16, out_idx=torch.empty((4, 8), dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError, match="k_scale must have shape"):
        K8 = K.float().to(torch.float8_e4m3fn)
        itk.indexer_topk_fused(Q, K8, W, kv, 16, k_scale=torch.ones(499, device="cuda"))
    with pytest.raises(ValueError, match="prior must be contiguous"):
        itk.indexer_topk_fused_prior(Q, K, W, kv, 16, torch.arange(0, 100, dtype=torch.int32, device="cuda")[::2])
    idx, sc = itk.indexer_topk_fused(Q, K, W, kv, 16)
    torch.cuda.synchronize()
    assert ((idx >= 0) & (idx < 500)).all()


def test_ragged_arguments_are_checked(itk):
    x = torch.randn(4, 256, device="cuda")
    rl = torch.full((4,), 256, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="scores must be contiguous"):
        itk.topk_ragged(x.t(), rl, 8)
    with pytest.raises(ValueError, match="scores must be contiguous"):
        itk.topk_ragged(x[:, :200], rl, 8)   # a padded view: rows are not 200 apart
    with pytest.raises(TypeError, match="scores must be torch.float32"):
        itk.topk_ragged(x.half(), rl, 8)
    with pytest.raises(TypeError, match="row_len must be torch.int32"):
        itk.topk_ragged(x, rl.long(), 8)
    with pytest.raises(ValueError, match="row_len must have shape"):
        itk.topk_ragged(x, rl[:2], 8)
    with pytest.raises(ValueError, match="out_idx must have shape"):
        itk.topk_ragged_noalloc(x, rl, 8, torch.empty((4, 4), dtype=torch.int32, device="cuda"))
    out = itk.topk_ragged(x, rl, 8).long()
    torch.cuda.synchronize()
    # the well-formed call: 8 distinct indices per row, none beaten by an unselected value
    assert (out.sort(dim=1).values.diff(dim=1) > 0).all() and ((out >= 0) & (out < 256)).all()
    sel = torch.zeros_like(x, dtype=torch.bool).scatter_(1, out, True)
    assert (x.gather(1, out).min(dim=1).values >= x.masked_fill(sel, -float("inf")).max(dim=1).values).all()
