"""Seeded synthetic inputs for online-softmax attention.

This module is shared by the tests and the benchmark.  It holds only input
preparation -- shapes, seeds, random draws and the rounding of f32 draws to the
stored input dtype -- and none of the attention arithmetic, so that the HIP
path and the CPU oracle can be fed identical bytes without sharing any code.

Recipe (the same for every workload):
  * ``numpy.random.default_rng(seed).standard_normal(shape, dtype=float32)``
    draws q, k, v and then dO, in that order, each of shape (H, N, D);
  * the f32 draws are rounded to nearest-even to the stored dtype (fp16 by
    numpy's cast, bf16 by the bit-level rule below);
  * varlen sequence lengths come from a separate
    ``default_rng(seed + 1).integers(lo, hi + 1)`` stream, drawn in order until
    the running total reaches the token budget; the last length is truncated
    so the total is exact (it may then be shorter than ``lo``; length-1
    sequences are legal, as the TIGA-lang varlen example shows).

The named workloads follow the attention workloads on the pages (TIGA-lang
"Attention and dense relations": N=1024, H=4, D=64 fp16 dense; a causal
triangular relation; a varlen causal block-diagonal relation) and the
rectangular SQ=8192 x SK=2048, HD=64 FP32 shape of the Vx issue "Chunked-dot
Reduce lowering" (evidence section).  Seeds follow the pages' examples where
one exists (0 for the dense example, 7 for the causal one, 20260821 for the
varlen one).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round f32 to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Inputs here are finite normal draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to f32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_dtype(x32: np.ndarray, dtype: str):
    """Return (stored, widened_f32): the stored array (f32, f16 or bf16 bits as
    uint16) and its exact widening to f32."""
    if dtype == "f32":
        s = np.ascontiguousarray(x32, dtype=np.float32)
        return s, s
    if dtype == "f16":
        s = x32.astype(np.float16)
        return s, s.astype(np.float32)
    if dtype == "bf16":
        s = f32_to_bf16_bits(x32)
        return s, bf16_bits_to_f32(s)
    raise ValueError(dtype)


def varlen_lengths(seed: int, total: int, lo: int, hi: int) -> List[int]:
    """Sequence lengths uniform on [lo, hi], drawn until ``total`` tokens."""
    rng = np.random.default_rng(seed)
    out: List[int] = []
    acc = 0
    while acc < total:
        L = int(rng.integers(lo, hi + 1))
        L = min(L, total - acc)
        out.append(L)
        acc += L
    return out


def cu_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


@dataclass
class Workload:
    name: str
    H: int
    n_q: int
    n_k: int
    D: int
    dtype: str
    causal: bool
    seed: int
    backward: bool = False
    lengths: Optional[List[int]] = None  # varlen only
    scale: Optional[float] = None  # default D^-1/2
    description: str = ""

    @property
    def varlen(self) -> bool:
        return self.lengths is not None

    @property
    def softmax_scale(self) -> float:
        return float(self.D) ** -0.5 if self.scale is None else float(self.scale)

    @property
    def cu_seqlens(self) -> Optional[np.ndarray]:
        return None if self.lengths is None else cu_from_lengths(self.lengths)


@dataclass
class Inputs:
    """Stored inputs (what the GPU receives) and their exact f32 widening."""
    w: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    q32: np.ndarray
    k32: np.ndarray
    v32: np.ndarray
    do32: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray] = field(default=None)


def make_inputs(w: Workload, with_grad: Optional[bool] = None) -> Inputs:
    """Draw q, k, v (and dO) for a workload, laid out (H, N, D)."""
    with_grad = w.backward if with_grad is None else with_grad
    rng = np.random.default_rng(w.seed)
    q32 = rng.standard_normal((w.H, w.n_q, w.D), dtype=np.float32)
    k32 = rng.standard_normal((w.H, w.n_k, w.D), dtype=np.float32)
    v32 = rng.standard_normal((w.H, w.n_k, w.D), dtype=np.float32)
    do32 = rng.standard_normal((w.H, w.n_q, w.D), dtype=np.float32) if with_grad else None
    q, qw = round_to_dtype(q32, w.dtype)
    k, kw = round_to_dtype(k32, w.dtype)
    v, vw = round_to_dtype(v32, w.dtype)
    if do32 is not None:
        do, dow = round_to_dtype(do32, w.dtype)
    else:
        do, dow = None, None
    return Inputs(w, q, k, v, do, qw, kw, vw, dow, w.cu_seqlens)


def _varlen_workload() -> Workload:
    seed = 20260821
    lengths = varlen_lengths(seed + 1, 16384, 37, 2048)
    total = sum(lengths)
    return Workload("varlen_causal_16k_h8_d64_f16", 8, total, total, 64, "f16", True, seed,
                    lengths=lengths,
                    description="varlen causal, lengths U[37,2048] to 16384 tokens, H=8, D=64, fp16")


WORKLOADS = {
    "dense_n128_h1_d64_f32": Workload(
        "dense_n128_h1_d64_f32", 1, 128, 128, 64, "f32", False, 0,
        description="dense forward, N=128, H=1, D=64, fp32"),
    "dense_n1024_h4_d64_f16": Workload(
        "dense_n1024_h4_d64_f16", 4, 1024, 1024, 64, "f16", False, 0, scale=0.125,
        description="dense forward, N=1024, H=4, D=64, fp16 (H,N,D), f32 accumulation"),
    "causal_n4096_h16_d128_bf16": Workload(
        "causal_n4096_h16_d128_bf16", 16, 4096, 4096, 128, "bf16", True, 7,
        description="causal forward, N=4096, H=16, D=128, bf16, f32 accumulation"),
    "varlen_causal_16k_h8_d64_f16": _varlen_workload(),
    "rect_sq8192_sk2048_h1_d64_f32_fwdbwd": Workload(
        "rect_sq8192_sk2048_h1_d64_f32_fwdbwd", 1, 8192, 2048, 64, "f32", False, 0,
        backward=True,
        description="dense rectangular SQ=8192 x SK=2048, H=1, D=64, fp32, forward + backward"),
}

# The order the workloads are listed in (index 0 is the small correctness case).
ORDER = list(WORKLOADS)

# Extra measurement shapes (not among the five above): the dense relation at the
# causal workload's size, where tile pruning (a dense-only approximation) has
# enough tiles per query block to act, and a decode-like split-KV shape.
EXTRA = {
    "dense_n4096_h16_d128_bf16": Workload(
        "dense_n4096_h16_d128_bf16", 16, 4096, 4096, 128, "bf16", False, 7,
        description="dense forward, N=4096, H=16, D=128, bf16 (tile-pruning measurement)"),
    # Few queries against long keys (decode-like): the forward splits the key
    # range over workgroups and merges the partial states in a second launch.
    "decode_q128_k16384_h8_d128_bf16": Workload(
        "decode_q128_k16384_h8_d128_bf16", 8, 128, 16384, 128, "bf16", False, 11,
        description="dense forward, 128 queries x 16384 keys, H=8, D=128, bf16 (split-KV measurement)"),
}
WORKLOADS.update(EXTRA)


# ------------------------------------------------------------------ CSR graphs
def csr_graph(seed: int, n_dst: int, n_src: int, mean_degree: float, max_degree: int,
              empty_frac: float = 0.02):
    """A seeded random CSR relation: heavy-tailed row degrees (Pareto, shape 2,
    scaled to `mean_degree`, clipped to `max_degree`), `empty_frac` of the rows
    with no edges, and sources drawn uniformly.  Returns int32 arrays
    (row_ptr (n_dst + 1,), col_idx (nnz,))."""
    rng = np.random.default_rng(seed)
    deg = np.floor((rng.pareto(2.0, size=n_dst) + 1.0) * (mean_degree / 2.0)).astype(np.int64)
    deg = np.clip(deg, 1, max_degree)
    deg[rng.random(n_dst) < empty_frac] = 0
    row_ptr = np.zeros(n_dst + 1, dtype=np.int64)
    np.cumsum(deg, out=row_ptr[1:])
    col_idx = rng.integers(0, n_src, size=int(row_ptr[-1]))
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def csr_inputs(seed: int, H: int, n_src: int, nnz: int, D: int, dtype: str):
    """Edge scores (H, nnz) f32 ~ N(0, 1) and values (H, n_src, D) ~ N(0, 1)
    rounded to dtype; returns (scores, v_stored, v_widened_f32)."""
    rng = np.random.default_rng(seed + 1)
    scores = rng.standard_normal((H, nnz), dtype=np.float32)
    v32 = rng.standard_normal((H, n_src, D), dtype=np.float32)
    v, vw = round_to_dtype(v32, dtype)
    return scores, v, vw


# The CSR measurement workload: 65536 rows over 65536 sources, mean degree 32.
CSR_WORKLOAD = {"name": "csr_n65536_deg32_h4_d64_f16", "seed": 4242, "n_dst": 65536,
                "n_src": 65536, "mean_degree": 32, "max_degree": 2048, "H": 4, "D": 64,
                "dtype": "f16"}
