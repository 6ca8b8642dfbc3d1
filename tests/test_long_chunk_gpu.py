"""The long-context prefill chunk: the last 8192 queries of a 2^20-token
prefill against FP8 keys with per-key scales, causal lengths, k = 2048 (the
shape of LiteTopK Sec. 4.1 "Sparse-Attention Kernel Benchmark" and Sec. 4.2,
Fig. 5(a)), in the launch configuration that the benchmark times.  Evenly
spaced rows, first and last included, are checked against the oracle with
the fused parity checks, in both scoring modes (FP8 keys widened to bf16,
and FP8 scoring against the quantized-query oracle)."""
import numpy as np
import pytest
import torch

import synth
from parity import check_fused_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chunk():
    return synth.long_context_chunk()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fp8_score", [False, True], ids=["widened", "fp8_scoring"])
def test_long_context_chunk_sampled_rows(itk, chunk, fp8_score):
    case = chunk
    case.flags = (case.flags | itk.FLAG_FP8_SCORE) if fp8_score else (case.flags & ~itk.FLAG_FP8_SCORE)
    Q, K, S, W, kv = itk.fused_tensors(case)
    idx, sc = itk.indexer_topk_fused(Q, K, W, kv, case.k, k_scale=S, flags=case.flags)
    torch.cuda.synchronize()
    rows = np.linspace(0, case.T - 1, 3).round().astype(np.int64)
    rec = check_fused_rows(case, rows, idx.cpu().numpy(), sc.cpu().numpy())
    print(f"long-context chunk {'fp8 scoring' if fp8_score else 'widened'}: rows {rows.tolist()} recall {rec.tolist()}")
    del Q, K, S, W, kv, idx, sc
