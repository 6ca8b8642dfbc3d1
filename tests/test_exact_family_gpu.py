"""Fused calls on inputs whose scores are exact in fp32 (small integers,
power-of-two weights and per-key scales; synth.gen_fused_exact): the kernel's
scores then equal the definition's whatever the summation order, so the index
sets and scores must equal the oracle's bit for bit, including which members
of a tied group at the k-th score are taken (the lower indices).  Ties are
frequent with small integers.  Every route runs: the staged head-rows scan,
the few-query scan (one and two queries), the single-head kernels, key
splits, candidate overflow, a view longer than the candidate buffer, and the
forced re-scoring route; every dtype pair, FP8 keys widened and FP8 scoring.
Lengths include 0, 1, k - 1, k, k + 1, N and two outside [0, N]."""
import numpy as np
import pytest
import torch

import synth
from parity import check_fused_exact

pytestmark = pytest.mark.gpu

T, N, K = 19, 9000, 300
KV = np.array([N, N - 1, 8000, K + 1, K, K - 1, 1, 0, 64, 65, 4500, N + 321, -9] +
              [N - 37 * i for i in range(6)], dtype=np.int32)

KNOBS = {"default": {}, "recovery": dict(force_route=1), "overflow": dict(capacity=K, rho=50.0),
         "splits": dict(splits=8), "long_view": dict(sample_stride=1, rho=1.0)}

# (q dtype, k dtype, H, D, fp8 scoring)
HEAD_ROWS = [(synth.BF16, synth.BF16, 64, 128, False), (synth.F16, synth.F16, 8, 256, False),
             (synth.F32, synth.F32, 40, 64, False), (synth.BF16, synth.FP8_E4M3, 33, 64, False),
             (synth.F16, synth.FP8_E4M3, 20, 128, False), (synth.BF16, synth.FP8_E4M3, 64, 128, True),
             (synth.F16, synth.FP8_E4M3, 24, 256, True)]
# (q dtype, k dtype, D, no ReLU)
SINGLE_HEAD = [(synth.BF16, synth.BF16, 128, False), (synth.F16, synth.F16, 256, True),
               (synth.F16, synth.FP8_E4M3, 64, False), (synth.BF16, synth.FP8_E4M3, 128, True)]


@pytest.fixture(autouse=True)
def _reset(itk):
    itk.reset_plan_opts()
    yield
    itk.reset_plan_opts()


def _run(itk, case, knobs):
    Q, K_, S, W, kv = itk.fused_tensors(case)
    itk.set_plan_opts(**knobs)
    idx, sc = itk.indexer_topk_fused(Q, K_, W, kv, case.k, k_scale=S, flags=case.flags)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("knob", list(KNOBS))
@pytest.mark.parametrize("qt,kt,H,D,fp8", HEAD_ROWS)
def test_head_rows_bit_exact(itk, qt, kt, H, D, fp8, knob):
    case = synth.gen_fused_exact(T, H, D, N, K, q_dtype=qt, k_dtype=kt, kv_len=KV, fp8_score=fp8,
                                 seed=H * 31 + D + fp8)
    idx, sc = _run(itk, case, KNOBS[knob])
    check_fused_exact(case, range(T), idx, sc)


@pytest.mark.parametrize("nq", [1, 2])
@pytest.mark.parametrize("qt,kt,H,D,fp8", HEAD_ROWS)
def test_few_queries_bit_exact(itk, qt, kt, H, D, fp8, nq):
    kv = np.array([N + 5, K - 3][:nq], np.int32)
    case = synth.gen_fused_exact(nq, H, D, N, K, q_dtype=qt, k_dtype=kt, kv_len=kv, fp8_score=fp8, seed=H + nq)
    idx, sc = _run(itk, case, {})
    check_fused_exact(case, range(nq), idx, sc)


@pytest.mark.parametrize("knob", list(KNOBS))
@pytest.mark.parametrize("qt,kt,D,no_relu", SINGLE_HEAD)
def test_single_head_bit_exact(itk, qt, kt, D, no_relu, knob):
    # 600 queries: two 512-query groups, the second ragged
    Tq = 600
    kv = np.resize(KV, Tq)
    kv[19:] = (np.arange(Tq - 19) * 53 % N + 200).astype(np.int32)
    case = synth.gen_fused_exact(Tq, 1, D, N, K, q_dtype=qt, k_dtype=kt, kv_len=kv, no_relu=no_relu, seed=D + no_relu)
    idx, sc = _run(itk, case, KNOBS[knob])
    check_fused_exact(case, range(Tq), idx, sc)


@pytest.mark.parametrize("P", [4, 8])
def test_gate_published_across_splits(itk, P):
    """Key splits with a loose sampled gate (rho = 50) and the row's best keys
    all in the first split: that split's own admitted keys raise its gate and
    publish it, and the other splits move up to it.  The result stays the
    oracle's exactly (the candidate counts are printed: on one box 2000 /
    3100 / 5900 per row at 4 / 8 / 16 splits, against 3500 / 5700 / 8700
    with the publication switched off)."""
    T_, N_, K_ = 8, 40000, 256
    case = synth.gen_fused_exact(T_, 64, 128, N_, K_, kv_len=np.full(T_, N_), seed=77 + P)
    span = -(-N_ // P)
    kf = synth.decode_reference_free(case.k_bits, case.k_dtype).reshape(N_, 128)
    kf[:span // 2] = np.abs(kf[:span // 2]) * 2  # strong keys at the start of split 0
    case.k_bits = synth.encode(kf.astype(np.float32), case.k_dtype)
    itk.set_plan_opts(splits=P, rho=50.0)
    Q, K, S, W, kv = itk.fused_tensors(case)
    cnt = torch.full((T_,), -1, dtype=torch.int32, device="cuda")
    itk.set_count_buffer(cnt)
    try:
        idx, sc = itk.indexer_topk_fused(Q, K, W, kv, K_, k_scale=S)
        torch.cuda.synchronize()
    finally:
        itk.set_count_buffer(None)
    check_fused_exact(case, range(T_), idx.cpu().numpy(), sc.cpu().numpy())
    c = cnt.cpu().numpy()
    print(f"P={P}: candidates per row {c.tolist()}")
