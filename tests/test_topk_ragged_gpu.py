"""topk_ragged on the GPU: bit-exact index sets against the CPU oracle.

Every test runs under each mapping of the selector: segments (view and scan
per segment, finish per row), row-local (one workgroup per row, sampled
steps) and row-local with the direct-exact steps for every row that fits the
on-chip stash (no view); rows longer than the row-local limit take the
segments either way."""
import numpy as np
import pytest
import torch

import synth
from parity import check_ragged_exact

pytestmark = pytest.mark.gpu


def _run(itk, case, routes=False):
    x = torch.from_numpy(case.scores).cuda()
    rl = torch.from_numpy(case.row_len).cuda()
    rb = None
    if routes:
        rb = torch.zeros(case.M, dtype=torch.int32, device="cuda")
        itk.set_route_buffer(rb)
    try:
        out = itk.topk_ragged(x, rl, case.k)
        torch.cuda.synchronize()
    finally:
        if routes:
            itk.set_route_buffer(None)
    return out.cpu().numpy(), (rb.cpu().numpy() if routes else None)


@pytest.fixture(autouse=True, params=[1, 2, 3], ids=["segments", "rowlocal", "direct"])
def route(request, itk):
    itk.reset_plan_opts()
    itk.set_plan_opts(ragged_route=request.param)
    yield request.param
    itk.reset_plan_opts()


def test_config2_bit_exact(itk):
    case = synth.ragged_config()
    out, routes = _run(itk, case, routes=True)
    check_ragged_exact(case, out)
    print("config2 routes:", np.bincount(routes, minlength=5).tolist())


@pytest.mark.parametrize("family", synth.RAGGED_FAMILIES)
def test_families_bit_exact(itk, family):
    lens = [20000, 2049, 2048, 2047, 1, 0, 4097, 131, 12345, 65536]
    case = synth.gen_ragged(len(lens), 65536, 2048, lens=lens, seed=17, family=family)
    out, _ = _run(itk, case)
    check_ragged_exact(case, out)


@pytest.mark.parametrize("pitch", [65536, 10001])
def test_lengths_outside_the_pitch_are_clamped(itk, pitch):
    """row_len > pitch reads the whole row, a negative row_len none of it
    (the operator contract: only valid entries are read); 10001 takes the
    scalar path."""
    lens = [pitch + 1, pitch + 100000, -1, -70000, pitch, 3000]
    case = synth.gen_ragged(len(lens), pitch, 2048, lens=lens, seed=23, family="config2")
    out, _ = _run(itk, case)
    check_ragged_exact(case, out)
    assert (out[2:4] == -1).all()


def test_small_k_and_odd_pitch(itk):
    # pitch not a multiple of 4 takes the scalar path
    case = synth.gen_ragged(7, 10001, 37, lens=[10001, 9000, 36, 37, 38, 5000, 3], seed=3, family="config2")
    out, _ = _run(itk, case)
    check_ragged_exact(case, out)


@pytest.mark.parametrize("force", [1, 2])
def test_forced_routes_match(itk, force, route):
    case = synth.ragged_config(seed=808, M=16)
    base, _ = _run(itk, case)
    itk.set_plan_opts(force_route=force, ragged_route=route)
    forced, routes = _run(itk, case, routes=True)
    check_ragged_exact(case, forced)
    assert np.array_equal(np.sort(base, axis=1), np.sort(forced, axis=1))
    assert (routes == (3 if force == 1 else 2)).all(), routes


def test_tiny_view_underfills_then_recovers(itk, route):
    # A huge stride with a low target rank underfills the primary boundary.
    case = synth.gen_ragged(8, 131072, 2048, seed=5, family="off_view")
    itk.set_plan_opts(sample_stride=2048, rho=1.0, rho1=1.01, ragged_route=route)
    out, routes = _run(itk, case, routes=True)
    check_ragged_exact(case, out)
    print("off_view routes:", routes.tolist())


def test_capacity_overflow_goes_exact(itk, route):
    case = synth.gen_ragged(4, 65536, 2048, seed=6, family="all_equal")
    itk.set_plan_opts(capacity=256, ragged_route=route)
    out, routes = _run(itk, case, routes=True)
    check_ragged_exact(case, out)
    assert (routes == 3).all()


def test_many_rows(itk):
    case = synth.gen_ragged(1024, 16384, 512, lens=np.random.default_rng(1).integers(0, 16385, 1024),
                            seed=8, family="config2")
    out, _ = _run(itk, case)
    check_ragged_exact(case, out)


def test_repeat_deterministic(itk):
    case = synth.ragged_config(seed=99, M=8)
    a, _ = _run(itk, case)
    for _ in range(5):
        b, _ = _run(itk, case)
        assert np.array_equal(np.sort(a, axis=1), np.sort(b, axis=1))


@pytest.mark.parametrize("M,family,k", [(1, "config2", 2048), (3, "config2", 2048), (2, "descending", 2048),
                                        (2, "gaussian", 64)])
def test_decode_rows_of_one_million(itk, M, family, k):
    """A few rows of 2^20 scores (decoding against a 1M context): the planner
    spreads each row over up to 64 segments; a descending row puts every top
    value in one segment, overflows its slices and takes the exact route.
    With k = 64 the view's sample rank would be below 32 at rho = 1.5, so
    the planner raises rho to 32 s / k = 64."""
    pitch = 1 << 20
    lens = np.array([pitch, pitch - 12345, pitch - 1][:M], dtype=np.int32)
    case = synth.gen_ragged(M, pitch, k, lens=lens, seed=900 + M, family=family)
    out, routes = _run(itk, case, routes=True)
    check_ragged_exact(case, out)
    if family == "descending":
        assert (routes == 3).all(), routes  # overflow -> exact route
