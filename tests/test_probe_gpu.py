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


def _fp8_dot(itk, a_pairs, b_pairs, acc=None):
    """Every output of one scaled FP8 MFMA (unit block scales) with every row
    of A equal to the vector a and every column of B equal to b: the dot
    product a . b (plus ``acc``, the accumulator input).  Every value given
    is exactly representable in e4m3fn."""
    a = np.zeros(64, np.float32)
    b = np.zeros(64, np.float32)
    for k, v in a_pairs:
        a[k] = v
    for k, v in b_pairs:
        b[k] = v
    A, B = np.tile(a, (32, 1)), np.tile(b[:, None], (1, 32))
    fa, fb = _frag_layout(A, B, 32)
    ta = torch.from_numpy(fa).to(torch.float8_e4m3fn).view(torch.uint8).cuda().contiguous()
    tb = torch.from_numpy(fb).to(torch.float8_e4m3fn).view(torch.uint8).cuda().contiguous()
    assert np.array_equal(torch.from_numpy(fa).to(torch.float8_e4m3fn).float().numpy(), fa), "not e4m3fn values"
    if acc is None:
        c = itk.debug_mfma(3, ta, tb).cpu().numpy()
    else:
        c = itk.debug_mfma(4, ta, tb, acc=torch.full((64, 16), acc, dtype=torch.float32, device="cuda")).cpu().numpy()
    assert (c == c[0, 0]).all()
    return float(c[0, 0])


def test_fp8_mfma_accumulation(itk):
    """The scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) adds each group
    of 8 consecutive products aligned to the group's largest (exponent E):
    every product is truncated toward zero to a multiple of 2^(E - 13), so a
    product below 2^(E - 13) vanishes; the group sums and the accumulator
    input are added at fp32 precision.  This is not an fp32 sum: on random
    operands the recursive-sum bound fails, and
    parity.fp8_mfma_alignment_error (the bound the FP8-scoring checks use)
    holds."""
    from parity import fp8_mfma_alignment_error
    # groups of 8: largest product 1 at k = 0, a product 2^-16 (2^-7 * 2^-9) at k
    for k, kept in [(1, False), (7, False), (8, True), (15, True), (16, True), (40, True), (63, True)]:
        got = _fp8_dot(itk, [(0, 1.0), (k, 2.0 ** -7)], [(0, 1.0), (k, 2.0 ** -9)]) - 1.0
        assert got == (2.0 ** -16 if kept else 0.0), (k, got)
    # the window: 2^-13 of the group's largest is kept, 2^-14 vanishes, either sign
    assert _fp8_dot(itk, [(0, 1.0), (1, 2.0 ** -6)], [(0, 1.0), (1, 2.0 ** -7)]) == 1.0 + 2.0 ** -13
    assert _fp8_dot(itk, [(0, 1.0), (1, 2.0 ** -6)], [(0, 1.0), (1, 2.0 ** -8)]) == 1.0
    assert _fp8_dot(itk, [(0, 1.0), (1, -2.0 ** -6)], [(0, 1.0), (1, 2.0 ** -7)]) == 1.0 - 2.0 ** -13
    assert _fp8_dot(itk, [(0, 1.0), (1, -2.0 ** -6)], [(0, 1.0), (1, 2.0 ** -8)]) == 1.0
    # truncation toward zero on the grid 2^(8 - 13) of a largest product 448 = 1.75 * 2^8
    assert _fp8_dot(itk, [(0, 448.0), (1, 1.0)], [(0, 1.0), (1, 0.109375)]) == 448.0 + 0.09375
    assert _fp8_dot(itk, [(0, 448.0), (1, 1.0)], [(0, 1.0), (1, 0.0546875)]) == 448.0 + 0.03125
    # the accumulator input is added at fp32 precision
    assert _fp8_dot(itk, [(0, 1.0), (8, 1.0)], [(0, 1.0), (8, 1.0)], acc=2.0 ** 20) == 2.0 ** 20 + 2.0
    assert _fp8_dot(itk, [(k, 2.0 ** -6) for k in range(8)], [(k, 2.0 ** -8) for k in range(8)], acc=1.0) \
        == 1.0 + 2.0 ** -11
    # random operands
    rng = np.random.default_rng(8)
    over_fp32 = 0
    for trial in range(24):
        A = (rng.standard_normal((32, 64)) * np.exp2(rng.integers(-6, 6, size=(32, 64)))).astype(np.float32)
        B = (rng.standard_normal((64, 32)) * np.exp2(rng.integers(-6, 6, size=(64, 32)))).astype(np.float32)
        Aq = torch.from_numpy(A).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
        Bq = torch.from_numpy(B).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
        fa, fb = _frag_layout(Aq.astype(np.float32), Bq.astype(np.float32), 32)
        ta = torch.from_numpy(fa).to(torch.float8_e4m3fn).view(torch.uint8).cuda().contiguous()
        tb = torch.from_numpy(fb).to(torch.float8_e4m3fn).view(torch.uint8).cuda().contiguous()
        got = itk.debug_mfma(3, ta, tb).cpu().numpy().astype(np.float64)
        prod = Aq[:, None, :] * Bq.T[None, :, :]                      # [row, col, k]
        err = np.abs(got - _expected_c(prod.sum(axis=2)))
        absum = np.abs(prod).sum(axis=2)
        n = 10  # 8 group sums, the accumulator input and the result
        bound = fp8_mfma_alignment_error(prod) + n * 2.0 ** -23 / (1 - n * 2.0 ** -23) * absum
        assert (err <= _expected_c(bound)).all(), f"trial {trial}: {np.max(err / _expected_c(bound)):.3g} x the bound"
        over_fp32 += int((err > _expected_c(64 * 2.0 ** -23 * absum)).sum())
    assert over_fp32 > 0, "the FP8 sums rounded like fp32 sums"


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
