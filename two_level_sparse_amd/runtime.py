"""Device-side state for decode steps through the libtls C ABI.

PyTorch allocates device memory and provides streams; all computation is in
the library's HIP kernels. A `Cache` holds one KV cache with its block
summaries and INT4 label cache (built once by tls_build_summaries); a
`Decoder` owns the per-step buffers and workspaces and enqueues one decode
step (tls_select_blocks -> tls_select_tokens -> tls_sparse_decode).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (TLS_WS_BLOCKS, TLS_WS_DECODE, TLS_WS_TOKENS, shape_of, tls_build_summaries, tls_select_blocks,
               tls_select_tokens, tls_sparse_decode, tls_workspace_size)


def _dev(x, dtype=None, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(x)) if isinstance(x, np.ndarray) else x
    if dtype is not None:
        t = t.view(dtype) if t.element_size() == torch.empty((), dtype=dtype).element_size() else t.to(dtype)
    return t.to(device, non_blocking=False).contiguous()


def bf16(x_bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> bf16 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).to(device)


class Cache:
    """KV cache [B,Hkv,N,row] (bf16) plus its summaries and label cache on the device."""

    def __init__(self, s, kv, label_ch, device="cuda"):
        self.s = s
        self.shape = shape_of(s)
        self.kv = kv if isinstance(kv, torch.Tensor) else bf16(kv, device)
        assert tuple(self.kv.shape) == (s.B, s.Hkv, s.N, s.row) and self.kv.dtype == torch.bfloat16
        self.label_ch = torch.as_tensor(np.ascontiguousarray(label_ch, dtype=np.int32)).to(device)
        self.summ = torch.empty((s.B, s.Hkv, s.NB, 2, s.D), dtype=torch.bfloat16, device=device)
        self.codes = torch.empty((s.B, s.Hkv, s.N, s.r // 2), dtype=torch.uint8, device=device)
        self.scale = torch.empty((s.B, s.Hkv, s.N), dtype=torch.float32, device=device)

    def build(self, stream=None):
        tls_build_summaries(self.shape, self.kv, self.label_ch, self.summ, self.codes, self.scale, stream)
        return self


class Decoder:
    """Per-step buffers; `step(q)` enqueues the three calls of one decode step."""

    def __init__(self, s, device="cuda"):
        self.s = s
        self.shape = shape_of(s)
        self.kb = min(s.Kb, s.NB)
        self.kt = min(s.Kt, self.kb * s.bs)
        self.block_idx = torch.empty((s.B, s.Hkv, self.kb), dtype=torch.int32, device=device)
        self.block_score = torch.empty((s.B, s.Hkv, s.NB), dtype=torch.float32, device=device)
        self.token_idx = torch.empty((s.B, s.Hkv, self.kt), dtype=torch.int32, device=device)
        self.out = torch.empty((s.B, s.Hq, s.DV), dtype=torch.float32, device=device)
        self.lse = torch.empty((s.B, s.Hq), dtype=torch.float32, device=device)
        self.ws_sizes = {w: tls_workspace_size(self.shape, w) for w in (TLS_WS_BLOCKS, TLS_WS_TOKENS, TLS_WS_DECODE)}
        if min(self.ws_sizes.values()) == 0:
            raise ValueError(f"invalid shape for libtls: {s}")
        # zero-filled: the decode workspace begins with self-resetting split counters
        self.ws = {w: torch.zeros(n, dtype=torch.uint8, device=device) for w, n in self.ws_sizes.items()}

    def select_blocks(self, q, cache, stream=None, keep_scores=False, block_idx=None):
        bi = self.block_idx if block_idx is None else block_idx
        tls_select_blocks(self.shape, q, cache.summ, bi, self.block_score if keep_scores else None,
                          self.ws[TLS_WS_BLOCKS], self.ws_sizes[TLS_WS_BLOCKS], stream)

    def select_tokens(self, q, cache, stream=None, block_idx=None):
        bi = self.block_idx if block_idx is None else block_idx
        tls_select_tokens(self.shape, q, cache.label_ch, cache.codes, cache.scale, bi, self.token_idx,
                          self.ws[TLS_WS_TOKENS], self.ws_sizes[TLS_WS_TOKENS], stream)

    def decode(self, q, kv_cache, stream=None, slot_map=None, slots=0, token_idx=None):
        ti = self.token_idx if token_idx is None else token_idx
        tls_sparse_decode(self.shape, q, kv_cache, slot_map, slots, ti, self.out, self.lse,
                          self.ws[TLS_WS_DECODE], self.ws_sizes[TLS_WS_DECODE], stream)

    def step(self, q, cache, stream=None, keep_scores=False):
        self.select_blocks(q, cache, stream, keep_scores)
        self.select_tokens(q, cache, stream)
        self.decode(q, cache.kv, stream)
        return self.out
