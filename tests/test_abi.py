"""The C-ABI library loads, exports every declared symbol, and validates its
arguments on the host (no GPU needed: invalid calls return before any HIP call)."""
import ctypes
import os
import re

import pytest

import indexer_exact_top_amd as itk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="itk.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)
    return sorted({n for n in names if n.startswith(("itk_", "topk_", "indexer_"))})


def test_every_declared_symbol_is_exported():
    lib = itk.lib()
    names = _declared_functions()
    assert "indexer_topk_fused" in names and "topk_ragged" in names
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"


def test_probes_live_in_their_own_library():
    """The test-only probes (itk_probe.h) are exported by libitk_probe.so
    and not by the product library."""
    names = _declared_functions("itk_probe.h")
    assert names == ["itk_debug_coarse", "itk_debug_fp8", "itk_debug_mfma", "itk_debug_stream_read"]
    probe = itk.probe_lib()
    for n in names:
        assert hasattr(probe, n), f"missing export {n}"
    product = ctypes.CDLL(itk.LIB_PATH)
    for n in names:
        assert not hasattr(product, n), f"{n} exported by the product library"


def test_status_strings():
    lib = itk.lib()
    assert lib.itk_status_string(0) == b"ok"
    assert lib.itk_status_string(3).startswith(b"workspace")


P = ctypes.c_void_p
FAKE = P(0x10000)  # never dereferenced: validation fails first


def test_ragged_validation():
    lib = itk.lib()
    ws = lib.topk_ragged_workspace_size(64, 131072, 2048)
    assert ws > 0
    assert lib.topk_ragged(None, 128, FAKE, 4, 8, FAKE, FAKE, ws, None) == 1
    # negative sizes are invalid; no rows or k == 0 is a complete call that
    # enqueues nothing (no pointer is read, so none is needed)
    assert lib.topk_ragged(FAKE, 128, FAKE, -1, 8, FAKE, FAKE, ws, None) == 1
    assert lib.topk_ragged(FAKE, 128, FAKE, 4, -1, FAKE, FAKE, ws, None) == 1
    assert lib.topk_ragged(FAKE, -1, FAKE, 4, 8, FAKE, FAKE, ws, None) == 1
    assert lib.topk_ragged(None, 128, None, 0, 8, None, None, 0, None) == 0
    assert lib.topk_ragged(None, 128, None, 4, 0, None, None, 0, None) == 0
    assert lib.topk_ragged_noalloc(None, 128, None, 0, 8, None, None) == 0
    assert lib.topk_ragged_noalloc(None, 128, None, 4, 0, None, None) == 0
    assert lib.topk_ragged_workspace_size(0, 128, 8) == 0
    # rows of pitch 0 are empty: only the padding is written, so out_idx is needed
    assert lib.topk_ragged(None, 0, None, 4, 8, None, None, 0, None) == 1
    assert lib.topk_ragged_noalloc(None, 0, None, 4, 8, None, None) == 1
    assert lib.topk_ragged(FAKE, 1 << 31, FAKE, 4, 8, FAKE, FAKE, ws, None) == 2
    need = lib.topk_ragged_workspace_size(4, 128, 8)
    assert lib.topk_ragged(FAKE, 128, FAKE, 4, 8, FAKE, None, need, None) == 3
    assert lib.topk_ragged(FAKE, 128, FAKE, 4, 8, FAKE, FAKE, need - 1, None) == 3
    assert lib.topk_ragged(FAKE, 128, FAKE, 4, 8, FAKE, P(0x10010), need, None) == 3  # misaligned


def test_fused_validation():
    lib = itk.lib()
    BF, F16, F32, FP8 = itk.BF16, itk.F16, itk.F32, itk.FP8_E4M3
    args = lambda **kw: dict(dict(Q=FAKE, qt=BF, K=FAKE, kt=BF, S=None, W=FAKE, kv=FAKE, T=4, H=8, D=64, N=1000,
                                  k=16, flags=0, oi=FAKE, os=FAKE, ws=FAKE, wsb=1 << 40), **kw)

    def call(a):
        return lib.indexer_topk_fused(a["Q"], a["qt"], a["K"], a["kt"], a["S"], a["W"], a["kv"], a["T"], a["H"],
                                      a["D"], a["N"], a["k"], a["flags"], a["oi"], a["os"], a["ws"], a["wsb"], None)

    assert call(args(Q=None)) == 1
    assert call(args(kt=FP8)) == 1                  # fp8 keys need a scale
    assert call(args(S=FAKE)) == 1                  # a scale only with fp8 keys
    # negative sizes are invalid; no queries or k == 0 is a complete call that
    # enqueues nothing, once the shape and dtypes pass the same checks
    assert call(args(T=-1)) == 1 and call(args(k=-1)) == 1 and call(args(N=-1)) == 1
    assert call(args(T=0, Q=None, K=None, W=None, kv=None, oi=None, os=None, ws=None, wsb=0)) == 0
    assert call(args(k=0, Q=None, K=None, W=None, kv=None, oi=None, os=None, ws=None, wsb=0)) == 0
    assert call(args(T=0, H=65)) == 2
    assert call(args(k=0, D=96)) == 2
    assert call(args(T=0, flags=1, H=2)) == 1
    # no keys: every row is empty, only the padding is written (outputs needed)
    assert call(args(N=0, oi=None)) == 1
    assert lib.indexer_topk_fused_workspace_size(0, 8, 64, 1000, 16, BF, BF, 0) == 0
    assert call(args(H=65)) == 2
    assert call(args(D=96)) == 2
    assert call(args(H=40, D=256)) == 2             # two head blocks need D <= 128
    assert call(args(qt=F32, kt=BF)) == 2           # unsupported pair
    assert call(args(qt=F32, kt=F32, H=40, D=128)) == 2
    assert call(args(flags=1, H=2)) == 1            # NO_RELU needs H == 1
    assert call(args(flags=4)) == 1
    assert call(args(flags=2)) == 2                 # FP8 scoring needs FP8 keys
    assert call(args(flags=2, kt=FP8, S=FAKE, qt=F32)) == 2
    assert call(args(flags=3, kt=FP8, S=FAKE, H=1)) == 2  # ... and at least two heads
    assert call(args(Q=P(0x10004))) == 1            # misaligned
    assert call(args(ws=None)) == 3
    assert call(args(wsb=16)) == 3


def test_fused_workspace_is_O_rows_k():
    lib = itk.lib()
    f = lambda T, N, k, H=64, D=128, qt=itk.BF16, kt=itk.BF16, fl=0: \
        lib.indexer_topk_fused_workspace_size(T, H, D, N, k, qt, kt, fl)
    # config 3 / 4 / 5 against their materialized fp32 score matrices
    c3 = f(2048, 133120, 2048)
    c4 = f(128, 1 << 20, 2048, kt=itk.FP8_E4M3)
    c5 = f(1024, 1 << 22, 4096, H=1, D=256, qt=itk.F16, kt=itk.F16, fl=1)
    assert 0 < c3 < 2048 * 133120 * 4 / 4
    assert 0 < c4 < 128 * (1 << 20) * 4 / 16
    assert 0 < c5 < 1024 * (1 << 22) * 4 / 32
    # bounded in the key count: the stored view of the sampled scores takes at
    # most the candidate buffer's bytes (cap = 4k entries of 8 B), else it is
    # not stored; linear in rows and k
    floor = f(2048, 1 << 24, 2048)  # view too long to store
    for N in (133120, 1 << 20, 1 << 22, 1 << 24):
        assert floor <= f(2048, N, 2048) <= floor + 2048 * 4 * 2048 * 8
    assert f(2048, 1 << 20, 2048) > floor  # a 2^20-key view is stored
    assert f(4096, 133120, 2048) == pytest.approx(2 * c3, rel=0.02)
    assert f(2048, 133120, 4096) < 2.1 * c3


def test_materialized_baseline_arithmetic():
    # The pages' materialization figures, which the O(rows*k) scratch avoids:
    # LiteTopK Sec. 1: an 8192-query chunk over 2^20 keys in fp32 is 32 GB.
    assert 8192 * (1 << 20) * 4 == 32 * (1 << 30)
    # StreamIndex abstract: [B=1, S=65536, H_I=64, T=S/4] fp32 is 256 GB.
    assert 1 * 65536 * 64 * (65536 // 4) * 4 == 256 * (1 << 30)


def test_plan_opts_validation():
    lib = itk.lib()
    bad = itk.PlanOpts(-1, 0, 0, 0, 0, 0, 0)
    assert lib.itk_set_plan_opts(ctypes.byref(bad)) == 1
    bad = itk.PlanOpts(0, 0, 0, 0, 0, 3, 0)
    assert lib.itk_set_plan_opts(ctypes.byref(bad)) == 1
    ok = itk.PlanOpts(0, 0, 0, 512, 0, 0, 0)
    assert lib.itk_set_plan_opts(ctypes.byref(ok)) == 0
    # rows of 2^20 scores take the segmented route, whose slices follow the capacity
    small = lib.topk_ragged_workspace_size(8, 1 << 20, 2048)
    assert lib.itk_set_plan_opts(None) == 0
    assert lib.topk_ragged_workspace_size(8, 1 << 20, 2048) > small
    # the row-local route (many rows of at most 2^18 scores) keeps its candidates on chip: its
    # scratch is the row order, 4 B per row
    assert lib.topk_ragged_workspace_size(1024, 131072, 2048) <= 4096
    assert lib.itk_set_plan_opts(ctypes.byref(itk.PlanOpts(0, 0, 0, 0, 0, 0, 3))) == 0  # row-local direct-exact
    assert lib.itk_set_plan_opts(ctypes.byref(itk.PlanOpts(0, 0, 0, 0, 0, 0, 4))) == 1
    assert lib.itk_set_plan_opts(None) == 0


def test_short_pitches_take_the_row_local_mapping_at_any_row_count():
    """A pitch that fits the on-chip stash (7680 scores) takes the row-local
    mapping however few rows there are; its only scratch is the row order
    (4 B per row, 256-byte aligned), where the segmented mapping needs
    per-segment candidate slices.  A longer pitch at few rows stays
    segmented."""
    lib = itk.lib()
    assert lib.itk_set_plan_opts(None) == 0
    for M in (1, 8, 64, 511):
        for pitch, k in ((7680, 2048), (4096, 64), (2048, 100), (7679, 8000)):
            assert lib.topk_ragged_workspace_size(M, pitch, k) == (4 * M + 255) // 256 * 256, (M, pitch, k)
    assert lib.topk_ragged_workspace_size(64, 7681, 2048) > 64 * 2048
    # the segments knob (route 1) keeps the segmented mapping for short pitches too
    assert lib.itk_set_plan_opts(ctypes.byref(itk.PlanOpts(0, 0, 0, 0, 0, 0, 1))) == 0
    try:
        assert lib.topk_ragged_workspace_size(64, 4096, 64) > 64 * 64
    finally:
        assert lib.itk_set_plan_opts(None) == 0


def test_history_sample_validation():
    lib = itk.lib()
    BF, F16 = itk.BF16, itk.F16
    wsz = lib.indexer_topk_fused_prior_workspace_size
    base = lib.indexer_topk_fused_workspace_size(64, 64, 128, 133120, 2048, BF, BF, 0)
    # no list: the strided view's plan; a list adds its gathered rows (O(n_prior))
    assert wsz(64, 64, 128, 133120, 2048, BF, BF, 0, 0) == base
    w6 = wsz(64, 64, 128, 133120, 2048, BF, BF, 0, 6144)
    assert base < w6 < base + 6144 * (256 + 8) + 64 * 4 + 4 * 256 + 2 * 64 * 2048 * 4
    assert wsz(64, 64, 128, 133120, 2048, BF, BF, 0, 1 << 16) > 0
    assert wsz(64, 64, 128, 133120, 2048, BF, BF, 0, (1 << 16) + 1) == 0   # above the largest list
    assert wsz(64, 64, 128, 133120, 2048, BF, BF, 0, -1) == 0
    assert wsz(64, 1, 256, 1 << 20, 2048, F16, F16, 1, 4096) == 0          # single-head path: no history
    call = lambda n, pr=FAKE, H=64, D=128, qt=BF, fl=0: lib.indexer_topk_fused_prior(
        FAKE, qt, FAKE, qt, None, FAKE, FAKE, 4, H, D, 1000, 16, fl, pr, n, FAKE, FAKE, FAKE, 1 << 40, None)
    assert call(-1) == 1
    assert call(5, pr=None) == 1
    assert lib.indexer_topk_fused_prior(None, BF, None, BF, None, None, None, 0, 64, 128, 1000, 16, 0, None, 5,
                                        None, None, None, 0, None) == 0     # no queries
    assert call((1 << 16) + 1) == 2
    assert call(64, H=1, D=256, qt=F16, fl=1) == 2
    # the list builder
    pw = lib.indexer_prior_workspace_size
    assert pw(2048, 2048, 133120, 6144) > 4 * 133120
    assert pw(16383, 2048, 1 << 20, 6144) > 0         # counts stay below 2^25
    assert pw(16384, 2048, 1 << 20, 6144) == 0
    assert pw(-1, 2048, 1000, 10) == 0 and pw(1, 0, 1000, 10) == 0 and pw(1, 8, 0, 10) == 0
    assert pw(1, 8, 1000, 0) == 0
    pf = lib.indexer_prior_from_topk
    need = pw(4, 8, 1000, 10)
    assert pf(None, 4, 8, 1000, 10, FAKE, FAKE, need, None) == 1
    assert pf(FAKE, 4, 8, 1000, 10, None, FAKE, need, None) == 1
    assert pf(FAKE, 4, 8, 1000, 10, FAKE, FAKE, need - 1, None) == 3
    assert pf(FAKE, 4, 8, 1 << 31, 10, FAKE, FAKE, need, None) == 2
