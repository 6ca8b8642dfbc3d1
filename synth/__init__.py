"""Seeded synthetic inputs for the fused Indexer-TopK and the ragged Top-k.

This module only draws inputs.  It holds none of the method's arithmetic: no
score, no selection, no binning.  Both the CPU oracle (``oracle/``) and the HIP
path (``indexer_exact_top_amd``) consume what it returns, and neither imports
the other.

The shapes and value distributions stand in for the pages' private workloads
(GLM-5.2 layer-1 indexer activations, Hy4-Preview captured score rows and
MSMARCO embeddings), which are not available:

* LiteTopK (arXiv 2607.11976), Sec. 2.1 Eq. (1): per-query head weights
  ``w[t,h]`` and FP8 indexer keys; Sec. 4.1: chunked prefill over a 1M context
  with k = 2048, and a retrieval benchmark with unit-norm embeddings.
* Sample-Guided Exact Top-K (arXiv 2609.08450), Sec. 2.1 operator contract:
  fp32 score rows at a padded pitch with ragged valid lengths, int32 output.

Every array is produced with ``numpy.random.Generator(PCG64(seed))``.  Narrow
formats are produced by round-to-nearest-even casts (torch for bf16 and
e4m3fn, numpy for fp16) and returned as raw bit patterns, so each consumer
decodes them itself.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32, BF16, F16, FP8_E4M3 = 0, 1, 2, 3
DTYPE_NAMES = {F32: "f32", BF16: "bf16", F16: "f16", FP8_E4M3: "fp8_e4m3"}
FLAG_NO_RELU = 1
FP8_E4M3_MAX = 448.0

__all__ = [
    "F32", "BF16", "F16", "FP8_E4M3", "FLAG_NO_RELU", "FusedCase", "RaggedCase",
    "gen_fused", "gen_fused_exact", "gen_ragged", "fused_config", "ragged_config", "csa_chunk", "CONFIGS",
    "prefill_chunk_pair",
    "encode", "decode_reference_free",
]


@dataclasses.dataclass
class FusedCase:
    """Inputs of one ``indexer_topk_fused`` call (host arrays).

    q_bits: [T, H, D] in ``q_dtype`` (float32 array for F32, uint16 bits for
    BF16/F16).  k_bits: [N, D] in ``k_dtype`` (float32, uint16 or uint8 bits).
    k_scale: [N] float32 per-key dequantisation factor (FP8 keys only).
    W: [T, H] float32.  kv_len: [T] int32 valid keys per query (<= N).
    """
    name: str
    T: int
    H: int
    D: int
    N: int
    k: int
    q_dtype: int
    k_dtype: int
    q_bits: np.ndarray
    k_bits: np.ndarray
    k_scale: Optional[np.ndarray]
    W: np.ndarray
    kv_len: np.ndarray
    flags: int = 0

    @property
    def sum_len(self) -> int:
        """Valid (query, key) pairs: lengths clamped to [0, N]."""
        return int(np.clip(self.kv_len.astype(np.int64), 0, self.N).sum())

    def flops(self) -> float:
        """Algorithmic multiply-add work of the contraction: 2*H*D per valid key."""
        return 2.0 * self.H * self.D * self.sum_len


@dataclasses.dataclass
class RaggedCase:
    """Inputs of one ``topk_ragged`` call: scores [M, pitch] fp32, row_len [M]."""
    name: str
    M: int
    pitch: int
    k: int
    scores: np.ndarray
    row_len: np.ndarray

    @property
    def sum_len(self) -> int:
        """Valid scores: lengths clamped to [0, pitch]."""
        return int(np.clip(self.row_len.astype(np.int64), 0, self.pitch).sum())


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def encode(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float32 ``x`` to ``dtype`` (RNE) and return the raw bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    import torch  # narrow casts only; torch is plumbing here
    t = torch.from_numpy(x)
    if dtype == BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == FP8_E4M3:
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(f"unknown dtype {dtype}")


def decode_reference_free(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Widen raw bits to float32 with torch/numpy casts (used by tests only)."""
    if dtype == F32:
        return np.asarray(bits, dtype=np.float32)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if dtype == BF16:
        return t.view(torch.bfloat16).float().numpy()
    if dtype == FP8_E4M3:
        return t.view(torch.float8_e4m3fn).float().numpy()
    raise ValueError(f"unknown dtype {dtype}")


def _normal_rows(rng, n, d, unit_norm, chunk=1 << 18):
    out = np.empty((n, d), dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        blk = rng.standard_normal((e - s, d), dtype=np.float32)
        if unit_norm:
            blk /= np.linalg.norm(blk, axis=1, keepdims=True)
        else:
            blk *= np.float32(1.0 / math.sqrt(d))
        out[s:e] = blk
    return out


def gen_fused(T, H, D, N, k, *, q_dtype=BF16, k_dtype=BF16, kv_len=None,
              seed=0, w_scale=None, no_relu=False, unit_norm=False,
              name="fused") -> FusedCase:
    """Draw one fused case.

    Q and K rows ~ N(0, I)/sqrt(D) (or unit-normalised Gaussians when
    ``unit_norm``).  W ~ U(0,1) * w_scale (default 1/H; 1 for NO_RELU with
    H = 1).  ``kv_len`` may be an int (all rows), an array, or None (= N).
    FP8 keys get a per-key scale max|K[j,:]|/448 and K/scale is cast to e4m3fn.
    """
    rng = _rng(seed)
    q = _normal_rows(rng, T * H, D, unit_norm).reshape(T, H, D)
    kf = _normal_rows(rng, N, D, unit_norm)
    if no_relu:
        W = np.ones((T, H), dtype=np.float32)
    else:
        ws = (1.0 / H) if w_scale is None else w_scale
        W = (rng.random((T, H), dtype=np.float32) * np.float32(ws)).astype(np.float32)
    if kv_len is None:
        kvl = np.full(T, N, dtype=np.int32)
    elif np.isscalar(kv_len):
        kvl = np.full(T, int(kv_len), dtype=np.int32)
    else:
        kvl = np.asarray(kv_len, dtype=np.int32)
    k_scale = None
    if k_dtype == FP8_E4M3:
        amax = np.abs(kf).max(axis=1)
        k_scale = np.where(amax > 0, amax / np.float32(FP8_E4M3_MAX), np.float32(1.0)).astype(np.float32)
        kf = kf / k_scale[:, None]
    return FusedCase(name=name, T=T, H=H, D=D, N=N, k=k, q_dtype=q_dtype, k_dtype=k_dtype,
                     q_bits=encode(q, q_dtype), k_bits=encode(kf, k_dtype), k_scale=k_scale,
                     W=W, kv_len=kvl, flags=FLAG_NO_RELU if no_relu else 0)


def gen_fused_exact(T, H, D, N, k, *, q_dtype=BF16, k_dtype=BF16, kv_len=None, seed=0,
                    no_relu=False, fp8_score=False, name="fused_exact") -> FusedCase:
    """A fused case whose scores are exact in fp32 whatever the summation order.

    Q and K entries are integers in [-4, 4] (exact in every input format,
    e4m3fn included), head weights are 1, 1/2 or 1/4 (signed when
    ``no_relu``), and FP8 keys get per-key scales 1/2, 1 or 2.  A head's dot
    product is then an integer of magnitude <= 16 D, and every partial sum
    of weighted heads is a multiple of 2^-3 below 2^19, so every fp32
    intermediate is exact and the scores, their ties and the Top-k are those
    of the exact definition.  With ``fp8_score`` the query entries are
    integers in [-7, 7] and every (query, head) row holds a +-7, so its
    quantization scale max|q| / 448 is 2^-6 and the quantized row is
    64 q (an e4m3fn value) exactly.  Small integers make ties frequent."""
    rng = _rng(seed)
    qmax = 7 if fp8_score else 4
    q = rng.integers(-qmax, qmax + 1, size=(T, H, D)).astype(np.float32)
    if fp8_score:
        pos = rng.integers(0, D, size=(T, H))
        sgn = np.where(rng.random((T, H)) < 0.5, -7.0, 7.0).astype(np.float32)
        np.put_along_axis(q, pos[..., None], sgn[..., None], axis=2)
    kf = rng.integers(-4, 5, size=(N, D)).astype(np.float32)
    W = (2.0 ** -rng.integers(0, 3, size=(T, H))).astype(np.float32)
    if no_relu:
        W *= np.where(rng.random((T, H)) < 0.5, -1.0, 1.0).astype(np.float32)
    if kv_len is None:
        kvl = np.full(T, N, dtype=np.int32)
    elif np.isscalar(kv_len):
        kvl = np.full(T, int(kv_len), dtype=np.int32)
    else:
        kvl = np.asarray(kv_len, dtype=np.int32)
    k_scale = None
    if k_dtype == FP8_E4M3:
        k_scale = (2.0 ** rng.integers(-1, 2, size=N)).astype(np.float32)
    flags = (FLAG_NO_RELU if no_relu else 0) | (2 if fp8_score else 0)
    return FusedCase(name=name, T=T, H=H, D=D, N=N, k=k, q_dtype=q_dtype, k_dtype=k_dtype,
                     q_bits=encode(q, q_dtype), k_bits=encode(kf, k_dtype), k_scale=k_scale,
                     W=W, kv_len=kvl, flags=flags)


# Ragged row families.  "config2" is the headline recipe: N(0,1) values, each
# valid entry replaced with probability 0.001 by N(4,1) (long tail), then
# floor(0.01*L) distinct target positions copy the value of a uniformly drawn
# source position of the same row (forced ties).  The others are adversarial.
RAGGED_FAMILIES = ("config2", "all_equal", "ascending", "descending", "few_values",
                   "signed_zero", "outlier", "off_view", "gaussian", "ties_at_k")


def _ragged_row(rng, L, k, family, row):
    if family in ("config2", "gaussian"):
        x = rng.standard_normal(L, dtype=np.float32)
        if family == "config2":
            tail = rng.random(L) < 0.001
            x[tail] = (rng.standard_normal(int(tail.sum()), dtype=np.float32) + np.float32(4.0))
            ndup = int(0.01 * L)
            if ndup:
                tgt = rng.choice(L, size=ndup, replace=False)
                src = rng.integers(0, L, size=ndup)
                x[tgt] = x[src]
        return x
    if family == "all_equal":
        return np.full(L, np.float32(0.5), dtype=np.float32)
    if family == "ascending":
        return np.arange(L, dtype=np.float32) * np.float32(1e-3)
    if family == "descending":
        return (L - np.arange(L, dtype=np.float32)) * np.float32(1e-3)
    if family == "few_values":
        return rng.integers(0, 4, size=L).astype(np.float32)
    if family == "signed_zero":
        x = np.where(rng.random(L) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        neg = rng.random(L) < 0.3
        x[neg] = -np.abs(rng.standard_normal(int(neg.sum()), dtype=np.float32)) - np.float32(1.0)
        return x
    if family == "outlier":
        x = rng.standard_normal(L, dtype=np.float32)
        x[rng.integers(0, L)] = np.float32(1e30)
        x[rng.integers(0, L)] = np.float32(-np.inf)
        x[rng.integers(0, L)] = np.float32(np.inf)
        return x
    if family == "off_view":
        # Large values only where (i // 16) is odd, so that a block-strided
        # sample of the row (any phase that lands on even blocks) misses them.
        x = rng.standard_normal(L, dtype=np.float32) - np.float32(10.0)
        blk = (np.arange(L) // 16) % 2 == 1
        x[blk] = rng.standard_normal(int(blk.sum()), dtype=np.float32) + np.float32(10.0)
        return x
    if family == "ties_at_k":
        # Many entries equal to the value that lands at rank k.
        x = rng.standard_normal(L, dtype=np.float32)
        x[rng.random(L) < 0.05] = np.float32(1.25)
        return x
    raise ValueError(family)


def gen_ragged(M, pitch, k, *, lens=None, seed=0, family="config2", name=None) -> RaggedCase:
    """Draw ``M`` ragged fp32 rows at ``pitch``; the padded tail holds -inf."""
    rng = _rng(seed)
    if lens is None:
        lens = np.full(M, pitch, dtype=np.int32)
    lens = np.asarray(lens, dtype=np.int32)
    scores = np.full((M, pitch), -np.inf, dtype=np.float32)
    fams = [family] * M if isinstance(family, str) else list(family)
    for r in range(M):
        L = min(max(int(lens[r]), 0), pitch)  # a length outside [0, pitch] fills the clamped part
        if L:
            scores[r, :L] = _ragged_row(rng, L, k, fams[r], r)
    return RaggedCase(name=name or f"ragged_{family if isinstance(family, str) else 'mix'}",
                      M=M, pitch=pitch, k=k, scores=scores, row_len=lens)


# ---------------------------------------------------------------------------
# The five workloads (sizes as given in the workload list of this project).
# ---------------------------------------------------------------------------

def fused_config(cfg: int, seed: Optional[int] = None, T: Optional[int] = None) -> FusedCase:
    """Configs 1, 3, 4, 5 (fused).  ``T`` optionally trims the query count
    (keeping the first T queries and their causal lengths)."""
    if cfg == 1:
        Tq = T or 64
        c = gen_fused(Tq, 8, 64, 4096, 256, q_dtype=F32, k_dtype=F32,
                      kv_len=np.arange(Tq, dtype=np.int32) + (4096 - 63),
                      seed=101 if seed is None else seed, w_scale=1.0, name="cfg1_tiny_fused")
    elif cfg == 3:
        Tq = T or 2048
        N = 131072 + 2048
        c = gen_fused(Tq, 64, 128, N, 2048, q_dtype=BF16, k_dtype=BF16,
                      kv_len=np.arange(Tq, dtype=np.int32) + 131073,
                      seed=303 if seed is None else seed, name="cfg3_dsa_prefill_chunk")
    elif cfg == 4:
        Tq = T or 128
        N = 1 << 20
        c = gen_fused(Tq, 64, 128, N, 2048, q_dtype=BF16, k_dtype=FP8_E4M3, kv_len=N,
                      seed=404 if seed is None else seed, name="cfg4_1m_subchunk_fp8k")
    elif cfg == 5:
        Tq = T or 1024
        N = 1 << 22
        c = gen_fused(Tq, 1, 256, N, 4096, q_dtype=F16, k_dtype=F16, kv_len=N,
                      seed=505 if seed is None else seed, no_relu=True, unit_norm=True,
                      name="cfg5_vector_retrieval")
    else:
        raise ValueError(f"config {cfg} is not a fused config")
    return c


def ragged_config(seed: int = 202, M: int = 64, pitch: int = 131072, k: int = 2048) -> RaggedCase:
    """Config 2: M rows, L ~ U{8192..131072}, k = 2048, config2 value family."""
    rng = _rng(seed)
    lens = rng.integers(8192, pitch + 1, size=M).astype(np.int32)
    return gen_ragged(M, pitch, k, lens=lens, seed=seed + 1, family="config2",
                      name="cfg2_standalone_ragged")


def csa_chunk(S: int, chunk: int, *, m: int = 4, k: int = 2048, H: int = 64, D: int = 128,
              start: Optional[int] = None, seed: int = 606) -> FusedCase:
    """One query chunk of a compressed-key (CSA) indexer step: a sequence of
    S tokens whose keys are compressed m to 1 (S/m key rows), the chunk's
    ``chunk`` query tokens starting at token ``start`` (default: the last
    chunk), H indexer heads of dimension D, bf16 Q and K ~ N(0,1)/sqrt(D),
    W ~ U(0,1)/H.  Token t sees the compressed keys whose m tokens are all at
    or before it: kv_len = floor((t + 1) / m), so the first m - 1 tokens of a
    sequence see no key (StreamIndex summary: V4-style CSA, H_I = 64, m = 4)."""
    N = S // m
    t0 = S - chunk if start is None else start
    kv = (np.arange(t0, t0 + chunk, dtype=np.int64) + 1) // m
    return gen_fused(chunk, H, D, N, k, q_dtype=BF16, k_dtype=BF16, kv_len=kv.astype(np.int32),
                     seed=seed, name=f"csa_chunk_S{S}_m{m}")


def long_context_chunk(T: int = 8192, N: int = 1 << 20, *, k: int = 2048, H: int = 64, D: int = 128,
                       seed: int = 808) -> FusedCase:
    """The last T query tokens of an N-token prefill (the shape of LiteTopK
    Sec. 4.1 "Sparse-Attention Kernel Benchmark" and Sec. 4.2, Fig. 5(a):
    1M context, chunk 8192, k = 2048): bf16 Q, FP8 e4m3
    keys with per-key scales, H indexer heads of dimension D, and causal
    lengths kv_len[t] = N - T + 1 + t (each query sees the keys up to and
    including its own token).  Values as in the other fused workloads."""
    kv = np.arange(N - T + 1, N + 1, dtype=np.int64)
    return gen_fused(T, H, D, N, k, q_dtype=BF16, k_dtype=FP8_E4M3, kv_len=kv.astype(np.int32), seed=seed,
                     name=f"long_context_chunk_T{T}_N{N}")


def prefill_chunk_pair(T, H, D, N, k, *, start: Optional[int] = None, n_hot: Optional[int] = None,
                       k_dtype=BF16, seed: int = 707, name: str = "prefill_chunk_pair"):
    """Two consecutive query chunks of one prefill over shared keys, with the
    temporal structure that LiteTopK Sec. 3.2 ("Sampling") relies on:
    adjacent chunks attend to the same prefix tokens.

    Every head h has a fixed direction u_h (a unit Gaussian vector).  Keys are
    N(0, I)/sqrt(D); ``n_hot`` of them (default 3k), drawn at random, each get
    a_j * u_h added for a random head h and a_j ~ U(0.5, 1.5), so that they
    score high for every query.  Query rows of both chunks are
    u_h + N(0, I)/sqrt(D); W ~ U(0,1)/H.  The current chunk's T query tokens
    sit at positions start .. start+T-1 (default: the last T keys) and the
    previous chunk's at the T positions before; a token at position p sees
    kv_len = p + 1 keys (capped at N).  Returns (previous, current) cases
    with the same K (and FP8 scales)."""
    rng = _rng(seed)
    n_hot = 3 * k if n_hot is None else n_hot
    u = _normal_rows(rng, H, D, True)
    kf = _normal_rows(rng, N, D, False)
    hot = rng.choice(N, size=min(n_hot, N), replace=False)
    kf[hot] += (rng.uniform(0.5, 1.5, size=hot.size)[:, None] * u[rng.integers(0, H, size=hot.size)]).astype(np.float32)
    k_scale = None
    if k_dtype == FP8_E4M3:
        amax = np.abs(kf).max(axis=1)
        k_scale = np.where(amax > 0, amax / np.float32(FP8_E4M3_MAX), np.float32(1.0)).astype(np.float32)
        kf = kf / k_scale[:, None]
    k_bits = encode(kf, k_dtype)
    start = N - T if start is None else start
    cases = []
    for c, p0 in enumerate((start - T, start)):
        q = (u[None, :, :] + _normal_rows(rng, T * H, D, False).reshape(T, H, D)).astype(np.float32)
        W = (rng.random((T, H), dtype=np.float32) * np.float32(1.0 / H)).astype(np.float32)
        kv = np.minimum(np.arange(p0, p0 + T, dtype=np.int64) + 1, N).astype(np.int32)
        cases.append(FusedCase(name=f"{name}_{'prev' if c == 0 else 'cur'}", T=T, H=H, D=D, N=N, k=k,
                               q_dtype=BF16, k_dtype=k_dtype, q_bits=encode(q, BF16), k_bits=k_bits,
                               k_scale=k_scale, W=W, kv_len=kv))
    return cases[0], cases[1]


CONFIGS = {
    1: "tiny fused: T=64 H=8 D=64 fp32, N=4096, kv_len=4033+t, k=256",
    2: "standalone ragged: M=64 pitch=131072 L~U[8192,131072] fp32, k=2048",
    3: "DSA prefill chunk: T=2048 H=64 D=128 bf16, N=133120, kv_len=131073+t, k=2048",
    4: "1M sub-chunk: T=128 H=64 D=128 bf16 Q, fp8 e4m3 K + per-key scale, N=2^20, k=2048",
    5: "vector retrieval: T=1024 N=2^22 D=256 fp16 unit-norm, H=1 no ReLU, k=4096",
}
