"""Both calls captured into a HIP graph (torch.cuda.graph) and replayed: the
library enqueues only kernels on the caller's stream (no allocation, no
memset, no host read-back), so a replay on new input contents must give what
an eager call gives on them.  Each test replays several times, with eager
work and synchronizations between the replays, and checks every replay."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_ragged_graph_replays(itk):
    cases = [synth.gen_ragged(16, 8192, 300, lens=np.linspace(0, 8192, 16).astype(np.int32), seed=s,
                              family=f) for s, f in ((31, "config2"), (32, "ties_at_k"))]
    xs = [torch.from_numpy(c.scores).cuda() for c in cases]
    rl = torch.from_numpy(cases[0].row_len).cuda()
    k = cases[0].k
    eager = [np.sort(itk.topk_ragged(x, rl, k).cpu().numpy(), axis=1) for x in xs]
    buf = xs[0].clone()
    out = torch.empty((16, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(itk.topk_ragged_workspace_size(16, 8192, k), dtype=torch.uint8, device="cuda")
    g = _capture(lambda: itk.topk_ragged(buf, rl, k, out_idx=out, workspace=ws,
                                         stream=torch.cuda.current_stream()))
    for rep in range(6):
        i = rep % 2
        buf.copy_(xs[i])
        out.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(out.cpu().numpy(), axis=1), eager[i]), f"replay {rep}"


@pytest.mark.parametrize("cfg", ["head_rows", "single_head"])
def test_fused_graph_replays(itk, cfg):
    if cfg == "head_rows":
        mk = lambda s: synth.gen_fused(24, 64, 128, 6000, 256, kv_len=np.arange(24) * 200 + 1000, seed=s)
    else:
        mk = lambda s: synth.gen_fused(40, 1, 128, 6000, 256, q_dtype=synth.F16, k_dtype=synth.F16,
                                       kv_len=np.arange(40) * 100 + 1000, seed=s, no_relu=True)
    cases = [mk(41), mk(42)]
    ts = [itk.fused_tensors(c) for c in cases]
    c0 = cases[0]
    eager = []
    for Q, K, S, W, kv in ts:
        i, s = itk.indexer_topk_fused(Q, K, W, kv, c0.k, k_scale=S, flags=c0.flags)
        eager.append((np.sort(i.cpu().numpy(), axis=1), np.sort(s.cpu().numpy(), axis=1)))
    Qb, Kb, Sb, Wb, kvb = [t.clone() if t is not None else None for t in ts[0]]
    oi = torch.empty((c0.T, c0.k), dtype=torch.int32, device="cuda")
    osc = torch.empty((c0.T, c0.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(itk.fused_workspace_size(c0.T, c0.H, c0.D, c0.N, c0.k, c0.q_dtype, c0.k_dtype, c0.flags),
                     dtype=torch.uint8, device="cuda")
    g = _capture(lambda: itk.indexer_topk_fused(Qb, Kb, Wb, kvb, c0.k, k_scale=Sb, flags=c0.flags, out_idx=oi,
                                                out_score=osc, workspace=ws, stream=torch.cuda.current_stream()))
    for rep in range(6):
        i = rep % 2
        Qb.copy_(ts[i][0])
        Kb.copy_(ts[i][1])
        Wb.copy_(ts[i][3])
        oi.fill_(-7)
        osc.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(oi.cpu().numpy(), axis=1), eager[i][0]), f"replay {rep}: indices"
        assert np.array_equal(np.sort(osc.cpu().numpy(), axis=1), eager[i][1]), f"replay {rep}: scores"


def test_history_sample_graph_replays(itk):
    """The list builder and the gated fused call captured together (as a
    prefill step would: build the next chunk's list, then run the chunk), six
    replays on alternating inputs, each equal to the eager calls."""
    pairs = [synth.prefill_chunk_pair(32, 64, 128, 9000, 256, seed=s) for s in (51, 52)]
    T, k, N = 32, 256, 9000
    kp = 3 * k
    ts = [(itk.fused_tensors(p), itk.fused_tensors(c)) for p, c in pairs]
    eager = []
    for (Qp, K, _, Wp, kvp), (Q, _, _, W, kv) in ts:
        prev_idx, _ = itk.indexer_topk_fused(Qp, K, Wp, kvp, k)
        prior = itk.prior_from_topk(prev_idx, N, kp)
        i, s = itk.indexer_topk_fused_prior(Q, K, W, kv, k, prior)
        eager.append((prev_idx.clone(), prior.cpu().numpy(), np.sort(i.cpu().numpy(), axis=1)))
    Kb = ts[0][0][1].clone()
    Qb, Wb, kvb = ts[0][1][0].clone(), ts[0][1][3].clone(), ts[0][1][4].clone()
    prev_b = eager[0][0].clone()
    prior_b = torch.empty(kp, dtype=torch.int32, device="cuda")
    pws = torch.empty(itk.prior_workspace_size(T, k, N, kp), dtype=torch.uint8, device="cuda")
    oi = torch.empty((T, k), dtype=torch.int32, device="cuda")
    osc = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(itk.fused_prior_workspace_size(T, 64, 128, N, k, synth.BF16, synth.BF16, 0, kp),
                     dtype=torch.uint8, device="cuda")

    def step():
        st = torch.cuda.current_stream()
        itk.prior_from_topk(prev_b, N, kp, out=prior_b, workspace=pws, stream=st)
        itk.indexer_topk_fused_prior(Qb, Kb, Wb, kvb, k, prior_b, out_idx=oi, out_score=osc, workspace=ws,
                                     stream=st)

    g = _capture(step)
    for rep in range(6):
        i = rep % 2
        Kb.copy_(ts[i][0][1])
        Qb.copy_(ts[i][1][0])
        Wb.copy_(ts[i][1][3])
        kvb.copy_(ts[i][1][4])
        prev_b.copy_(eager[i][0])
        oi.fill_(-7)
        prior_b.fill_(-9)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(prior_b.cpu().numpy(), eager[i][1]), f"replay {rep}: list"
        assert np.array_equal(np.sort(oi.cpu().numpy(), axis=1), eager[i][2]), f"replay {rep}: indices"


def test_noalloc_graph_replays(itk):
    """topk_ragged_noalloc captured and replayed: its static scratch carries
    state only within a call."""
    cases = [synth.gen_ragged(16, 8192, 300, lens=np.linspace(0, 8192, 16).astype(np.int32), seed=s,
                              family="config2") for s in (61, 62)]
    xs = [torch.from_numpy(c.scores).cuda() for c in cases]
    rl = torch.from_numpy(cases[0].row_len).cuda()
    k = cases[0].k
    eager = [np.sort(itk.topk_ragged(x, rl, k).cpu().numpy(), axis=1) for x in xs]
    buf = xs[0].clone()
    out = torch.empty((16, k), dtype=torch.int32, device="cuda")
    g = _capture(lambda: itk.topk_ragged_noalloc(buf, rl, k, out_idx=out, stream=torch.cuda.current_stream()))
    for rep in range(6):
        i = rep % 2
        buf.copy_(xs[i])
        out.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(out.cpu().numpy(), axis=1), eager[i]), f"replay {rep}"
