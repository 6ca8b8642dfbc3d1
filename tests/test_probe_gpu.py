"""GPU probes of the building blocks the kernels rely on (in-bounds, one wave)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _frag_layout(A, B, per):
    """Per-lane operand fragments of a 32x32 MFMA: lane l holds row (l % 32)
    of A and column (l % 32) of B, at k = per*(l // 32) .. + per - 1."""
    a = np.stack([A[l % 32, per * (l // 32): per * (l // 32) + per] for l in range(64)])
    b = np.stack([B[per * (l // 32): per * (l // 32) + per, l % 32] for l in range(64)])
    return a, b


def _expected_c(C):
    """Accumulator layout: lane l, register r -> row 8(r//4) + 4(l//32) + r%4, column l % 32."""
    out = np.empty((64, 16))
    for l in range(64):
        for r in range(16):
            out[l, r] = C[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32]
    return out


@pytest.mark.parametrize("mtype,per", [(0, 8), (1, 8), (2, 1)])
def test_mfma_lane_layout(itk, mtype, per):
    rng = np.random.default_rng(mtype)
    K = 2 * per
    A = rng.integers(-4, 5, size=(32, K)).astype(np.float32)
    B = rng.integers(-4, 5, size=(K, 32)).astype(np.float32)
    a, b = _frag_layout(A, B, per)
    if mtype == 2:
        ta = torch.from_numpy(a.reshape(64).copy()).cuda()
        tb = torch.from_numpy(b.reshape(64).copy()).cuda()
    else:
        dt = torch.bfloat16 if mtype == 0 else torch.float16
        ta = torch.from_numpy(a).to(dt).cuda().contiguous()
        tb = torch.from_numpy(b).to(dt).cuda().contiguous()
    c = itk.debug_mfma(mtype, ta, tb).cpu().numpy()
    np.testing.assert_array_equal(c, _expected_c(A @ B))


def test_fp8_widening_is_exact(itk):
    codes = torch.arange(256, dtype=torch.uint8).cuda()
    bf, hf = itk.debug_fp8(codes)
    ref = oracle.decode(np.arange(256, dtype=np.uint8), synth.FP8_E4M3)
    got_bf = oracle.decode(bf.cpu().numpy().view(np.uint16), synth.BF16)
    got_hf = oracle.decode(hf.cpu().numpy().view(np.uint16), synth.F16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got_bf), nan) and np.array_equal(np.isnan(got_hf), nan)
    assert np.array_equal(got_bf[~nan], ref[~nan]) and np.array_equal(got_hf[~nan], ref[~nan])


def test_coarse_key_monotone_and_endpoints(itk):
    rng = np.random.default_rng(0)
    x = np.sort(np.concatenate([rng.standard_normal(1500).astype(np.float32) * 10,
                                np.array([-np.inf, np.inf, 0.0, -0.0, 1e-30, -1e-30, 7e4, -7e4], np.float32),
                                rng.standard_normal(540).astype(np.float32) * 1e-4]))
    key, ep = itk.debug_coarse(torch.from_numpy(x).cuda())
    key = key.cpu().numpy()
    ep = ep.cpu().numpy()
    assert (np.diff(key) >= 0).all(), "coarse key must be monotone"
    # the endpoint of bin b admits exactly the values whose coarse key is >= b
    for b in range(0, 2048, 7):
        assert np.array_equal(x >= ep[b], key >= b), f"bin {b}"
