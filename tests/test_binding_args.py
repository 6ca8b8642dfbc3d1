"""The binding checks every tensor before it reaches the C ABI (CPU: these
checks run before any GPU call).  The kernels read each buffer as a dense
row-major array of one element type, so a host tensor, a wrong dtype, a
wrong shape or a strided view is rejected with a message that names the
argument, instead of being read wrongly."""
import pytest
import torch

import indexer_exact_top_amd as itk


def test_host_tensors_are_rejected_before_any_gpu_call():
    Q = torch.zeros(4, 8, 64, dtype=torch.bfloat16)
    K = torch.zeros(100, 64, dtype=torch.bfloat16)
    W = torch.zeros(4, 8)
    kv = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="Q must be on a HIP device"):
        itk.indexer_topk_fused(Q, K, W, kv, 16)
    with pytest.raises(ValueError, match="scores must be on a HIP device"):
        itk.topk_ragged(torch.zeros(4, 128), torch.zeros(4, dtype=torch.int32), 8)
    with pytest.raises(ValueError, match="prev_idx must be on a HIP device"):
        itk.prior_from_topk(torch.zeros(4, 8, dtype=torch.int32), 100, 24)
    with pytest.raises(TypeError, match="must be a torch tensor"):
        itk.topk_ragged([[1.0]], torch.zeros(1, dtype=torch.int32), 1)
