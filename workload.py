"""Seeded synthetic inputs for the two-level sparse-attention decode step.

This module only draws and lays out inputs; it holds none of the method's
arithmetic. Both the fp64 oracle (``oracle/``) and the HIP path
(``two_level_sparse_amd``) are fed from it, and neither imports the other.

Workloads follow the decode settings the AsyncTLS pages describe (long-context
decode with GQA and MLA attention, contexts from about 30k to 128k tokens; page
"AsyncTLS: Efficient Generative LLM Inference with Asynchronous Two-level
Sparse Attention", sections 1, 4). The pages evaluate on LongBench/RULER with
trained models; those are replaced here by seeded synthetic tensors of the
same shapes: N(0,1) queries, keys and values rounded to bf16, with a few fixed
key channels scaled x8 as outlier channels.

Layouts (row-major, all bf16 values are carried as uint16 bit patterns):
  q   [B, Hq, D]
  kv  [B, Hkv, N, row]   row = D + DV for GQA (K then V); row = D for MLA,
                          where V is the first DV entries of K.
  label_ch [Hkv, r] int32, ascending.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Shape:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    DV: int
    v_is_k_prefix: bool
    N: int
    bs: int
    r: int
    Kb: int
    Kt: int
    n_outlier: int
    seed: int
    steps: int = 0          # staggered (offloaded) decode steps; 0 = single step
    sm: float | None = None # softmax scale; None = 1/sqrt(D)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def NB(self) -> int:
        return (self.N + self.bs - 1) // self.bs

    @property
    def row(self) -> int:
        return self.D if self.v_is_k_prefix else self.D + self.DV

    @property
    def v_off(self) -> int:
        return 0 if self.v_is_k_prefix else self.D

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D) if self.sm is None else float(self.sm)

    @property
    def pairs(self) -> int:
        return self.B * self.Hkv

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


# The five decode workloads. Seeds are 1000 + workload number.
CONFIGS = {
    "c1_8k_gqa8": Shape("c1_8k_gqa8", B=1, Hq=8, Hkv=1, D=128, DV=128, v_is_k_prefix=False,
                        N=8192, bs=64, r=16, Kb=16, Kt=256, n_outlier=4, seed=1001),
    "c2_32k_gqa": Shape("c2_32k_gqa", B=4, Hq=32, Hkv=8, D=128, DV=128, v_is_k_prefix=False,
                        N=32768, bs=64, r=16, Kb=64, Kt=2048, n_outlier=8, seed=1002),
    "c3_128k_gqa": Shape("c3_128k_gqa", B=8, Hq=64, Hkv=8, D=128, DV=128, v_is_k_prefix=False,
                         N=131072, bs=64, r=16, Kb=128, Kt=4096, n_outlier=8, seed=1003),
    "c4_64k_mla": Shape("c4_64k_mla", B=16, Hq=128, Hkv=1, D=576, DV=512, v_is_k_prefix=True,
                        N=65536, bs=64, r=32, Kb=64, Kt=2048, n_outlier=0, seed=1004),
    "c5_256k_offload": Shape("c5_256k_offload", B=4, Hq=32, Hkv=8, D=128, DV=128,
                             v_is_k_prefix=False, N=262144, bs=64, r=16, Kb=128, Kt=4096,
                             n_outlier=8, seed=1005, steps=64),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(s: Shape) -> np.ndarray:
    """The key channels scaled x8, shared by all heads (a separate seeded stream)."""
    if s.n_outlier == 0:
        return np.zeros(0, dtype=np.int64)
    return np.random.default_rng(s.seed + 7).permutation(s.D)[: s.n_outlier]


def gen_q(s: Shape) -> np.ndarray:
    """Query of the decode step: [B, Hq, D] bf16 bits, N(0,1)."""
    rng = np.random.default_rng(np.random.SeedSequence([s.seed, 0]))
    return f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D), dtype=np.float32))


def gen_kv_pair(s: Shape, b: int, h: int, out: np.ndarray | None = None) -> np.ndarray:
    """Cached rows of one (batch, kv-head) pair: [N, row] bf16 bits.

    Keys are N(0,1) with the outlier channels multiplied by 8 (exact in fp32);
    values (GQA only) are N(0,1). Each pair has its own seeded stream, so any
    pair can be regenerated alone.
    """
    rng = np.random.default_rng(np.random.SeedSequence([s.seed, 1, b, h]))
    k = rng.standard_normal((s.N, s.D), dtype=np.float32)
    oc = outlier_channels(s)
    if oc.size:
        k[:, oc] *= np.float32(8.0)
    if out is None:
        out = np.empty((s.N, s.row), dtype=np.uint16)
    out[:, : s.D] = f32_to_bf16_bits(k)
    del k
    if not s.v_is_k_prefix:
        v = rng.standard_normal((s.N, s.DV), dtype=np.float32)
        out[:, s.D:] = f32_to_bf16_bits(v)
    return out


def gen_kv(s: Shape, threads: int | None = None) -> np.ndarray:
    """The whole cache [B, Hkv, N, row] bf16 bits (one seeded stream per pair)."""
    kv = np.empty((s.B, s.Hkv, s.N, s.row), dtype=np.uint16)
    jobs = [(b, h) for b in range(s.B) for h in range(s.Hkv)]
    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(lambda bh: gen_kv_pair(s, bh[0], bh[1], kv[bh[0], bh[1]]), jobs))
    return kv


CALIB_TOKENS = 4096


def label_channels(s: Shape, kv_first_batch: np.ndarray | None = None) -> np.ndarray:
    """Label channels per kv head: [Hkv, r] int32, ascending.

    Offline channel choice in the Double-Sparsity manner: for kv head h, the r
    key channels with the largest mean |K| over the first CALIB_TOKENS tokens
    of batch 0 (lower channel index first on equal means). ``kv_first_batch``
    may pass the [Hkv, N, row] rows of batch 0 to skip regenerating them.
    """
    out = np.empty((s.Hkv, s.r), dtype=np.int32)
    n = min(s.N, CALIB_TOKENS)
    for h in range(s.Hkv):
        rows = kv_first_batch[h] if kv_first_batch is not None else gen_kv_pair(s, 0, h)
        k = np.abs(bf16_bits_to_f64(rows[:n, : s.D]))
        mean = k.mean(axis=0)
        order = np.lexsort((np.arange(s.D), -mean))
        out[h] = np.sort(order[: s.r])
    return out


def drift_queries(s: Shape, q0: np.ndarray, steps: int) -> np.ndarray:
    """Queries of a run of decode steps: [steps, B, Hq, D] bf16 bits.

    q_0 is the step's query; q_t = sqrt(D) * u / |u| with u = q_{t-1} + 0.1*eps,
    eps ~ N(0, I), per head row, computed in float64 and rounded to bf16 via
    float32. The sqrt(D) factor keeps the N(0,1) scale of the entries.
    """
    rng = np.random.default_rng(np.random.SeedSequence([s.seed, 2]))
    qs = np.empty((steps,) + q0.shape, dtype=np.uint16)
    qs[0] = q0
    for t in range(1, steps):
        u = bf16_bits_to_f64(qs[t - 1]) + 0.1 * rng.standard_normal(q0.shape)
        u *= math.sqrt(s.D) / np.linalg.norm(u, axis=-1, keepdims=True)
        qs[t] = f32_to_bf16_bits(u.astype(np.float32))
    return qs


def small_shape(name="small", B=2, Hq=8, Hkv=2, D=128, DV=128, v_is_k_prefix=False,
                N=1000, bs=64, r=16, Kb=4, Kt=96, n_outlier=4, seed=7, steps=0) -> Shape:
    """A shape the oracle finishes in well under a second (ragged last block by default)."""
    return Shape(name, B=B, Hq=Hq, Hkv=Hkv, D=D, DV=DV, v_is_k_prefix=v_is_k_prefix, N=N, bs=bs,
                 r=r, Kb=Kb, Kt=Kt, n_outlier=n_outlier, seed=seed, steps=steps)
