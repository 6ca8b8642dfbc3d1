"""Python binding of the itk C ABI (include/itk.h): argument marshalling only.

Every step of the fused Indexer-TopK and of the ragged Top-k runs in the HIP
kernels of ``libitk.so``; this module only turns torch device tensors into
pointers, allocates outputs and workspaces with torch (plumbing), and passes
the current HIP stream.  There is no CPU fallback: the calls raise when the
library or a GPU is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libitk.so")
PROBE_LIB_PATH = os.path.join(HERE, "libitk_probe.so")

F32, BF16, F16, FP8_E4M3 = 0, 1, 2, 3
FLAG_NO_RELU = 1
FLAG_FP8_SCORE = 2  # FP8 keys: quantize Q per (query, head) row and score on the FP8 matrix cores
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "hip error", 5: "scratch limit"}
RAGGED_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None
_probe_lib = None


class ITKError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({STATUS.get(status, '?')})")
        self.status = status


class PlanOpts(ctypes.Structure):
    _fields_ = [("sample_stride", ctypes.c_int32), ("rho", ctypes.c_float), ("rho1", ctypes.c_float),
                ("capacity", ctypes.c_int32), ("splits", ctypes.c_int32), ("force_route", ctypes.c_int32),
                ("ragged_route", ctypes.c_int32)]


def lib():
    """Load libitk.so (built by ``build.py``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run indexer_exact_top_amd/build.py (hipcc, gfx950)")
        # torch first: the library then binds to the HIP runtime that torch
        # loaded (both name libamdhip64.so.7), so that device pointers and
        # streams from torch are valid in it
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
        L.topk_ragged_workspace_size.argtypes = [I32, I64, I32]
        L.topk_ragged_workspace_size.restype = SZ
        L.topk_ragged.argtypes = [P, I64, P, I32, I32, P, P, SZ, P]
        L.topk_ragged.restype = ctypes.c_int
        L.topk_ragged_noalloc.argtypes = [P, I64, P, I32, I32, P, P]
        L.topk_ragged_noalloc.restype = ctypes.c_int
        L.indexer_topk_fused_workspace_size.argtypes = [I32, I32, I32, I64, I32, ctypes.c_int, ctypes.c_int, U32]
        L.indexer_topk_fused_workspace_size.restype = SZ
        L.indexer_topk_fused.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P, P, P, I32, I32, I32, I64, I32, U32,
                                         P, P, P, SZ, P]
        L.indexer_topk_fused.restype = ctypes.c_int
        L.indexer_topk_fused_prior_workspace_size.argtypes = [I32, I32, I32, I64, I32, ctypes.c_int, ctypes.c_int,
                                                              U32, I32]
        L.indexer_topk_fused_prior_workspace_size.restype = SZ
        L.indexer_topk_fused_prior.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P, P, P, I32, I32, I32, I64, I32,
                                               U32, P, I32, P, P, P, SZ, P]
        L.indexer_topk_fused_prior.restype = ctypes.c_int
        L.indexer_prior_workspace_size.argtypes = [I32, I32, I64, I32]
        L.indexer_prior_workspace_size.restype = SZ
        L.indexer_prior_from_topk.argtypes = [P, I32, I32, I64, I32, P, P, SZ, P]
        L.indexer_prior_from_topk.restype = ctypes.c_int
        L.itk_status_string.argtypes = [ctypes.c_int]
        L.itk_status_string.restype = ctypes.c_char_p
        L.itk_last_hip_error.argtypes = []
        L.itk_last_hip_error.restype = ctypes.c_char_p
        L.itk_set_plan_opts.argtypes = [ctypes.POINTER(PlanOpts)]
        L.itk_set_plan_opts.restype = ctypes.c_int
        L.itk_set_route_buffer.argtypes = [P, I32]
        L.itk_set_route_buffer.restype = ctypes.c_int
        L.itk_set_count_buffer.argtypes = [P, I32]
        L.itk_set_count_buffer.restype = ctypes.c_int
        L.itk_profile_enable.argtypes = [I32]
        L.itk_profile_enable.restype = ctypes.c_int
        L.itk_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32),
                                       ctypes.POINTER(ctypes.c_char_p), I32]
        L.itk_profile_read.restype = I32
        _lib = L
    return _lib


def probe_lib():
    """Load libitk_probe.so, the test-only probes of the device building
    blocks (include/itk_probe.h); raise if it is missing."""
    global _probe_lib
    if _probe_lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: run indexer_exact_top_amd/build.py (hipcc, gfx950)")
        lib()  # torch and the HIP runtime first, as for the product library
        L = ctypes.CDLL(PROBE_LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        for name in ("itk_debug_mfma", "itk_debug_fp8", "itk_debug_coarse", "itk_debug_stream_read"):
            getattr(L, name).restype = ctypes.c_int
        L.itk_debug_mfma.argtypes = [I32, P, P, P, P]
        L.itk_debug_fp8.argtypes = [P, P, P, I32, P]
        L.itk_debug_coarse.argtypes = [P, P, P, I32, P]
        L.itk_debug_stream_read.argtypes = [P, ctypes.c_uint64, P, I32, P]
        _probe_lib = L
    return _probe_lib


def require_gpu():
    """Raise unless the HIP library loads and a GPU is visible."""
    import torch
    lib()
    if not torch.cuda.is_available():
        raise RuntimeError("no HIP device visible: the itk kernels need an MI355X (gfx950)")


def _ptr(t) -> Optional[int]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        if status == 4:  # ITK_ERR_HIP: name the runtime error
            what = f"{what} [{lib().itk_last_hip_error().decode()}]"
        raise ITKError(status, what)


def _need(t, name: str, dtypes, shape=None, device=None):
    """Checks that ``t`` is a contiguous device tensor of one of ``dtypes``
    (and of ``shape`` / on ``device`` when given): the kernels read every
    buffer as a dense row-major array of that element type."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's tensors are on {device}")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major without gaps)")


def _dtype_code(t) -> int:
    import torch
    m = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.float8_e4m3fn: FP8_E4M3}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


# ------------------------------------------------------------------ ragged
def topk_ragged_workspace_size(M: int, pitch: int, k: int) -> int:
    return int(lib().topk_ragged_workspace_size(M, pitch, k))


def topk_ragged(scores, row_len, k: int, out_idx=None, workspace=None, stream=None):
    """Exact Top-k of each ragged fp32 row; returns int32 [M, k] (set order, -1 pad)."""
    import torch
    _need(scores, "scores", torch.float32)
    if scores.dim() != 2:
        raise ValueError(f"scores must be [M, pitch], got shape {tuple(scores.shape)}")
    M, pitch = scores.shape
    dev = scores.device
    _need(row_len, "row_len", torch.int32, (M,), dev)
    if out_idx is None:
        out_idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    _need(out_idx, "out_idx", torch.int32, (M, k), dev)
    if workspace is None:
        workspace = torch.empty(max(1, topk_ragged_workspace_size(M, pitch, k)), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    st = lib().topk_ragged(_ptr(scores), pitch, _ptr(row_len), M, k, _ptr(out_idx), _ptr(workspace),
                           workspace.numel(), _stream(stream))
    _check(st, "topk_ragged")
    return out_idx


def topk_ragged_noalloc(scores, row_len, k: int, out_idx, stream=None):
    """topk_ragged with the library's static scratch (no workspace, nothing
    allocated by the call; ``out_idx`` [M, k] int32 must be given)."""
    import torch
    _need(scores, "scores", torch.float32)
    if scores.dim() != 2:
        raise ValueError(f"scores must be [M, pitch], got shape {tuple(scores.shape)}")
    M, pitch = scores.shape
    _need(row_len, "row_len", torch.int32, (M,), scores.device)
    _need(out_idx, "out_idx", torch.int32, (M, k), scores.device)
    st = lib().topk_ragged_noalloc(_ptr(scores), pitch, _ptr(row_len), M, k, _ptr(out_idx), _stream(stream))
    _check(st, "topk_ragged_noalloc")
    return out_idx


# ------------------------------------------------------------------- fused
def fused_workspace_size(T, H, D, N, k, q_t, k_t, flags=0) -> int:
    return int(lib().indexer_topk_fused_workspace_size(T, H, D, N, k, q_t, k_t, flags))


def _fused_inputs(Q, K, W, kv_len, k_scale):
    """Validates the fused inputs; returns (T, H, D, N, q_t, k_t)."""
    import torch
    _need(Q, "Q", (torch.bfloat16, torch.float16, torch.float32))
    if Q.dim() != 3:
        raise ValueError(f"Q must be [T, H, D], got shape {tuple(Q.shape)}")
    T, H, D = Q.shape
    dev = Q.device
    _need(K, "K", (torch.bfloat16, torch.float16, torch.float32, torch.float8_e4m3fn), None, dev)
    if K.dim() != 2 or K.shape[1] != D:
        raise ValueError(f"K must be [N, {D}], got shape {tuple(K.shape)}")
    N = K.shape[0]
    _need(W, "W", torch.float32, (T, H), dev)
    _need(kv_len, "kv_len", torch.int32, (T,), dev)
    if k_scale is not None:
        _need(k_scale, "k_scale", torch.float32, (N,), dev)
    return T, H, D, N, _dtype_code(Q), _dtype_code(K)


def _fused_outputs(T, k, dev, out_idx, out_score):
    import torch
    if out_idx is None:
        out_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if out_score is None:
        out_score = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(out_idx, "out_idx", torch.int32, (T, k), dev)
    _need(out_score, "out_score", torch.float32, (T, k), dev)
    return out_idx, out_score


def indexer_topk_fused(Q, K, W, kv_len, k: int, k_scale=None, flags: int = 0, out_idx=None, out_score=None,
                       workspace=None, stream=None):
    """Fused indexer score + exact Top-k.  Q [T,H,D], K [N,D] (bf16/f16/f32 or
    float8_e4m3fn with k_scale [N]), W [T,H] fp32, kv_len [T] int32.
    Returns (out_idx int32 [T,k], out_score fp32 [T,k])."""
    import torch
    T, H, D, N, q_t, k_t = _fused_inputs(Q, K, W, kv_len, k_scale)
    out_idx, out_score = _fused_outputs(T, k, Q.device, out_idx, out_score)
    if workspace is None:
        workspace = torch.empty(max(1, fused_workspace_size(T, H, D, N, k, q_t, k_t, flags)),
                                dtype=torch.uint8, device=Q.device)
    _need(workspace, "workspace", torch.uint8, None, Q.device)
    st = lib().indexer_topk_fused(_ptr(Q), q_t, _ptr(K), k_t, _ptr(k_scale), _ptr(W), _ptr(kv_len), T, H, D, N,
                                  k, flags, _ptr(out_idx), _ptr(out_score), _ptr(workspace), workspace.numel(),
                                  _stream(stream))
    _check(st, "indexer_topk_fused")
    return out_idx, out_score


def fused_prior_workspace_size(T, H, D, N, k, q_t, k_t, flags, n_prior) -> int:
    return int(lib().indexer_topk_fused_prior_workspace_size(T, H, D, N, k, q_t, k_t, flags, n_prior))


def indexer_topk_fused_prior(Q, K, W, kv_len, k: int, prior, k_scale=None, flags: int = 0, out_idx=None,
                             out_score=None, workspace=None, stream=None):
    """indexer_topk_fused with a history sample: ``prior`` is an int32 device
    tensor of key indices (the previous chunk's most frequent keys)."""
    import torch
    T, H, D, N, q_t, k_t = _fused_inputs(Q, K, W, kv_len, k_scale)
    n_prior = int(prior.numel()) if prior is not None else 0
    if prior is not None:
        _need(prior, "prior", torch.int32, (n_prior,), Q.device)
    out_idx, out_score = _fused_outputs(T, k, Q.device, out_idx, out_score)
    if workspace is None:
        workspace = torch.empty(max(1, fused_prior_workspace_size(T, H, D, N, k, q_t, k_t, flags, n_prior)),
                                dtype=torch.uint8, device=Q.device)
    _need(workspace, "workspace", torch.uint8, None, Q.device)
    st = lib().indexer_topk_fused_prior(_ptr(Q), q_t, _ptr(K), k_t, _ptr(k_scale), _ptr(W), _ptr(kv_len), T, H, D,
                                        N, k, flags, _ptr(prior), n_prior, _ptr(out_idx), _ptr(out_score),
                                        _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "indexer_topk_fused_prior")
    return out_idx, out_score


def prior_workspace_size(T_prev, k, N, k_prime) -> int:
    return int(lib().indexer_prior_workspace_size(T_prev, k, N, k_prime))


def prior_from_topk(prev_idx, N: int, k_prime: int, out=None, workspace=None, stream=None):
    """The k_prime most frequent keys of the previous chunk's lists
    ``prev_idx`` (int32 [T_prev, k], device); returns int32 [k_prime]."""
    import torch
    _need(prev_idx, "prev_idx", torch.int32)
    if prev_idx.dim() != 2:
        raise ValueError(f"prev_idx must be [T_prev, k], got shape {tuple(prev_idx.shape)}")
    T_prev, k = prev_idx.shape
    if out is None:
        out = torch.empty(k_prime, dtype=torch.int32, device=prev_idx.device)
    _need(out, "out", torch.int32, (k_prime,), prev_idx.device)
    if workspace is None:
        workspace = torch.empty(max(1, prior_workspace_size(T_prev, k, N, k_prime)), dtype=torch.uint8,
                                device=prev_idx.device)
    _need(workspace, "workspace", torch.uint8, None, prev_idx.device)
    st = lib().indexer_prior_from_topk(_ptr(prev_idx), T_prev, k, N, k_prime, _ptr(out), _ptr(workspace),
                                       workspace.numel(), _stream(stream))
    _check(st, "indexer_prior_from_topk")
    return out


def fused_tensors(case, device="cuda"):
    """Move a host case (raw bit arrays + dtype codes) to device tensors."""
    import torch

    def as_t(bits, code):
        t = torch.from_numpy(np.ascontiguousarray(bits))
        if code == F32:
            return t.to(device)
        if code == FP8_E4M3:
            return t.to(device).view(torch.float8_e4m3fn)
        t = t.view(torch.int16).to(device)
        return t.view(torch.bfloat16 if code == BF16 else torch.float16)

    Q = as_t(case.q_bits, case.q_dtype)
    K = as_t(case.k_bits, case.k_dtype)
    S = None if case.k_scale is None else torch.from_numpy(case.k_scale).to(device)
    W = torch.from_numpy(np.ascontiguousarray(case.W)).to(device)
    kv = torch.from_numpy(np.ascontiguousarray(case.kv_len, dtype=np.int32)).to(device)
    return Q, K, S, W, kv


# ------------------------------------------------------------------ knobs
def set_plan_opts(sample_stride=0, rho=0.0, rho1=0.0, capacity=0, splits=0, force_route=0, ragged_route=0):
    o = PlanOpts(sample_stride, rho, rho1, capacity, splits, force_route, ragged_route)
    _check(lib().itk_set_plan_opts(ctypes.byref(o)), "itk_set_plan_opts")


def reset_plan_opts():
    _check(lib().itk_set_plan_opts(None), "itk_set_plan_opts")


def set_route_buffer(t=None):
    import torch
    if t is not None:
        _need(t, "route buffer", torch.int32)
    _check(lib().itk_set_route_buffer(_ptr(t), 0 if t is None else t.numel()), "itk_set_route_buffer")


def set_count_buffer(t=None):
    import torch
    if t is not None:
        _need(t, "count buffer", torch.int32)
    _check(lib().itk_set_count_buffer(_ptr(t), 0 if t is None else t.numel()), "itk_set_count_buffer")


def profile_enable(on: bool = True):
    _check(lib().itk_profile_enable(1 if on else 0), "itk_profile_enable")


def profile_read():
    """{stage: (total_ms, launches)} since the last read."""
    n = 16
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    names = (ctypes.c_char_p * n)()
    k = lib().itk_profile_read(ms, cnt, names, n)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(k) if cnt[i]}


# ------------------------------------------------------------ test probes
def debug_mfma(mtype: int, a_frags, b_frags, acc=None):
    """One 32x32 MFMA on per-lane fragments; returns float32 [64, 16]
    (mtype 4: the FP8 MFMA onto the accumulator values ``acc`` [64, 16])."""
    import torch
    c = torch.empty((64, 16), dtype=torch.float32, device=a_frags.device) if acc is None else acc.clone()
    _check(probe_lib().itk_debug_mfma(mtype, _ptr(a_frags), _ptr(b_frags), _ptr(c), _stream(None)), "itk_debug_mfma")
    return c


def debug_fp8(codes):
    import torch
    bf = torch.empty(codes.numel(), dtype=torch.int16, device=codes.device)
    hf = torch.empty(codes.numel(), dtype=torch.int16, device=codes.device)
    _check(probe_lib().itk_debug_fp8(_ptr(codes), _ptr(bf), _ptr(hf), codes.numel(), _stream(None)), "itk_debug_fp8")
    return bf, hf


def debug_coarse(x):
    import torch
    n = x.numel()
    key = torch.empty(n, dtype=torch.int32, device=x.device)
    ep = torch.empty(n, dtype=torch.float32, device=x.device)
    _check(probe_lib().itk_debug_coarse(_ptr(x), _ptr(key), _ptr(ep), n, _stream(None)), "itk_debug_coarse")
    return key, ep


def debug_stream_read(x, blocks: int = 2048, out=None, stream=None):
    """Streaming read of the bytes of tensor x (max per workgroup into out)."""
    import torch
    if out is None:
        out = torch.empty(blocks, dtype=torch.float32, device=x.device)
    _check(probe_lib().itk_debug_stream_read(_ptr(x), x.numel() * x.element_size(), _ptr(out), blocks, _stream(stream)),
           "itk_debug_stream_read")
    return out
