"""Device-side state for decode steps through the libtls C ABI.

PyTorch allocates device memory and provides streams; all computation is in
the library's HIP kernels. A `Cache` holds one KV cache with its block
summaries and INT4 label cache (built once by tls_build_summaries); a
`Decoder` owns the per-step buffers and workspaces and enqueues one decode
step (tls_select -> tls_sparse_decode; tls_select is tls_select_blocks and
tls_select_tokens in one call).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (TLS_WS_BLOCKS, TLS_WS_DECODE, TLS_WS_SELECT, TLS_WS_STEP, TLS_WS_TOKENS, shape_of, tls_append_kv,
               tls_build_summaries, tls_decode_step, tls_decode_step_status, tls_select, tls_select_blocks,
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
        self.summ = torch.empty((s.B, s.Hkv, summ_pair_elems(s.NB, s.D)), dtype=torch.bfloat16, device=device)
        self.codes = torch.empty((s.B, s.Hkv, s.N, s.r // 2), dtype=torch.uint8, device=device)
        self.scale = torch.empty((s.B, s.Hkv, s.N), dtype=torch.float32, device=device)

    def build(self, stream=None):
        tls_build_summaries(self.shape, self.kv, self.label_ch, self.summ, self.codes, self.scale, stream)
        return self


def summ_pair_elems(nblocks, D):
    """bf16 elements of one pair's block summaries (tile-fragment order: whole
    tiles of 16 blocks, each block's Kmax and Kmin rows of D channels)."""
    return (nblocks + 15) // 16 * 16 * 2 * D


class GrowingCache:
    """A KV cache allocated for `capacity` tokens per sequence that grows at
    decode time: `append(rows)` writes new rows after the current length and
    updates the summaries and label cache of the blocks they fall in
    (tls_append_kv). Every per-sequence buffer is strided by `capacity`;
    `shape` describes the current length."""

    def __init__(self, s, kv, label_ch, capacity, device="cuda"):
        assert capacity >= s.N
        self.s, self.capacity, self.n = s, int(capacity), s.N
        nb_cap = (self.capacity + s.bs - 1) // s.bs
        self.kv = torch.zeros((s.B, s.Hkv, self.capacity, s.row), dtype=torch.bfloat16, device=device)
        self.kv[:, :, : s.N] = kv if isinstance(kv, torch.Tensor) else bf16(kv, device)
        self.label_ch = torch.as_tensor(np.ascontiguousarray(label_ch, dtype=np.int32)).to(device)
        self.summ = torch.zeros((s.B, s.Hkv, summ_pair_elems(nb_cap, s.D)), dtype=torch.bfloat16, device=device)
        self.codes = torch.zeros((s.B, s.Hkv, self.capacity, s.r // 2), dtype=torch.uint8, device=device)
        self.scale = torch.zeros((s.B, s.Hkv, self.capacity), dtype=torch.float32, device=device)

    @property
    def shape(self):
        return shape_of(self.s.with_(N=self.n), self.capacity)

    def build(self, stream=None):
        tls_build_summaries(self.shape, self.kv, self.label_ch, self.summ, self.codes, self.scale, stream)
        return self

    def append(self, rows, stream=None):
        """rows: [B, Hkv, n, row] bf16 device tensor (contiguous)."""
        n = rows.shape[2]
        tls_append_kv(self.shape, rows.contiguous(), n, self.kv, self.label_ch, self.summ, self.codes, self.scale,
                      stream)
        self.n += n
        return self


class Decoder:
    """Per-step buffers; `step(q)` enqueues the three calls of one decode step.
    `outputs` may supply the output tensors (e.g. views of larger buffers)."""

    def __init__(self, s, device="cuda", outputs=None):
        self.s = s
        self.shape = shape_of(s)
        self.kb = min(s.Kb, s.NB)
        self.kt = min(s.Kt, self.kb * s.bs)
        o = outputs or {}
        self.block_idx = o.get("block_idx", torch.empty((s.B, s.Hkv, self.kb), dtype=torch.int32, device=device))
        self.block_score = o.get("block_score", torch.empty((s.B, s.Hkv, s.NB), dtype=torch.float32, device=device))
        self.token_idx = o.get("token_idx", torch.empty((s.B, s.Hkv, self.kt), dtype=torch.int32, device=device))
        self.out = o.get("out", torch.empty((s.B, s.Hq, s.DV), dtype=torch.float32, device=device))
        self.lse = o.get("lse", torch.empty((s.B, s.Hq), dtype=torch.float32, device=device))
        self.ws_sizes = {w: tls_workspace_size(self.shape, w)
                         for w in (TLS_WS_BLOCKS, TLS_WS_TOKENS, TLS_WS_SELECT, TLS_WS_DECODE, TLS_WS_STEP)}
        if self.ws_sizes[TLS_WS_BLOCKS] == 0 or self.ws_sizes[TLS_WS_DECODE] == 0:
            raise ValueError(f"invalid shape for libtls: {s}")
        # (a zero TOKENS/SELECT size: more candidates than the token stage takes; select_tokens then fails;
        # a zero STEP size: a shape the one-launch step does not cover)
        # zero-filled: the one-launch step's workspace, and the counters at the start of the
        # attention's, must start cleared (every call leaves them so)
        self.ws = {w: torch.zeros(max(n, 256), dtype=torch.uint8, device=device) for w, n in self.ws_sizes.items()}
        self.one_launch = self.ws_sizes[TLS_WS_STEP] > 0

    # `shape`: the calls' shape when it differs from the decoder's (a growing
    # cache: current length and capacity; Kb' and Kt' must not change)
    def select_blocks(self, q, cache, stream=None, keep_scores=False, block_idx=None, shape=None):
        bi = self.block_idx if block_idx is None else block_idx
        tls_select_blocks(shape or self.shape, q, cache.summ, bi, self.block_score if keep_scores else None,
                          self.ws[TLS_WS_BLOCKS], self.ws_sizes[TLS_WS_BLOCKS], stream)

    def select_tokens(self, q, cache, stream=None, block_idx=None, shape=None):
        bi = self.block_idx if block_idx is None else block_idx
        tls_select_tokens(shape or self.shape, q, cache.label_ch, cache.codes, cache.scale, bi, self.token_idx,
                          self.ws[TLS_WS_TOKENS], self.ws_sizes[TLS_WS_TOKENS], stream)

    def select(self, q, cache, stream=None, shape=None):
        """Both selection stages (block_idx and token_idx) in one call."""
        tls_select(shape or self.shape, q, cache.summ, cache.label_ch, cache.codes, cache.scale, self.block_idx,
                   self.token_idx, self.ws[TLS_WS_SELECT], self.ws_sizes[TLS_WS_SELECT], stream)

    def decode(self, q, kv_cache, stream=None, slot_map=None, slots=0, token_idx=None, shape=None):
        ti = self.token_idx if token_idx is None else token_idx
        tls_sparse_decode(shape or self.shape, q, kv_cache, slot_map, slots, ti, self.out, self.lse,
                          self.ws[TLS_WS_DECODE], self.ws_sizes[TLS_WS_DECODE], stream)

    def step_one_launch(self, q, cache, stream=None, shape=None):
        """The whole step in one launch (tls_decode_step; shapes it covers)."""
        tls_decode_step(shape or self.shape, q, cache.summ, cache.label_ch, cache.codes, cache.scale, cache.kv,
                        self.block_idx, self.token_idx, self.out, self.lse, self.ws[TLS_WS_STEP],
                        self.ws_sizes[TLS_WS_STEP], stream)

    def step_status(self, stream=None):
        """Raises if a one-launch step abandoned work (synchronises `stream`)."""
        tls_decode_step_status(self.ws[TLS_WS_STEP], stream)

    def step(self, q, cache, stream=None, keep_scores=False, one_launch=False):
        """One decode step over `cache` (a Cache or GrowingCache).
        one_launch=True runs tls_decode_step (shapes it covers) in place of the
        separate calls; the separate calls are the default, being the faster
        of the two on the 128k GQA step (68.7 us against 77-79 us)."""
        sh = cache.shape if isinstance(cache, GrowingCache) else None
        if one_launch and not self.one_launch:
            raise ValueError("tls_decode_step does not cover this shape")
        if one_launch and not keep_scores:
            self.step_one_launch(q, cache, stream, shape=sh)
            return self.out
        if keep_scores:  # the block scores go to self.block_score
            self.select_blocks(q, cache, stream, keep_scores, shape=sh)
            self.select_tokens(q, cache, stream, shape=sh)
        else:
            self.select(q, cache, stream, shape=sh)
        self.decode(q, cache.kv, stream, shape=sh)
        return self.out


class StaggeredDecoder:
    """Staggered decode steps over a KV cache held in pinned host memory.

    Step t (AsyncTLS pages, section 2B): the token stage and the attention use
    M_{t-1}, the blocks chosen at step t-1, which are resident on the device,
    while the next selection is prepared on two side streams:
      stage stream: stage 1 for step t (M_t, from q_t and the block summaries);
      copy stream:  tls_prefetch_delta -- T_t = M_t minus the resident blocks,
                    evictions, and the host->device copies of T_t, which also
                    writes the slot map of step t+1.
    The main stream of step t+1 waits for those copies. The copy stream of step
    t waits for the main stream of step t-1 (so no slot or map entry that a
    running kernel reads is ever written) and for M_t. The stage stream of step
    t waits for the main stream of step t-1 only, so stage 1 runs under the
    copies of step t-1; M_t rotates over three buffers, and the buffer it
    overwrites (M_{t-3}) was last read by the token stage of step t-2 and the
    prefetch of step t-3, both finished before the main stream of step t-1
    started.

    `cache` holds the summaries and label cache on the device (its `kv` is not
    read); `host_kv` is the full cache [B,Hkv,Ns,row] bf16 in pinned memory, Ns
    >= s.N its allocated length. With Ns > s.N the cache can grow:
    `append(rows)` adds tokens between steps (host rows, index, resident
    slots); `cache` then holds its index at the capacity's strides (a
    GrowingCache).
    """

    def __init__(self, s, cache, host_kv, q0, device="cuda", copy_mode=None, stagger=True, streams=None):
        """streams: (stage, copy) streams to use instead of two of its own (the
        layers of a LayeredDecoder share theirs)."""
        self.s = s
        self.capacity = int(host_kv.shape[2])
        self.n = s.N
        s_cap = s.with_(N=self.capacity)
        # stagger=False: the baseline without staggering -- each step selects
        # M_t, moves T_t and then attends over tokens of M_t, in order on the
        # caller's stream (the transfers are the same; their time is not hidden)
        self.stagger = stagger
        self.cache = cache
        self.host_kv = host_kv
        # buffers and workspaces for the largest length (Kb' and Kt' do not change as it grows)
        self.dec = Decoder(s_cap, device)
        self.kb = self.dec.kb
        self.cap = 2 * self.kb
        self.dev_cache = torch.empty((s.B, s.Hkv, self.cap, s.bs, s.row), dtype=torch.bfloat16, device=device)
        self.maps = [torch.full((s.B, s.Hkv, s_cap.NB), -1, dtype=torch.int32, device=device) for _ in range(2)]
        # M_t lives in mbuf[t % 3]; M_{-1} (the prologue's selection) in mbuf[2]
        self.mbuf = [torch.empty((s.B, s.Hkv, self.kb), dtype=torch.int32, device=device) for _ in range(3)]
        if streams is None:
            streams = (torch.cuda.Stream(device=device), torch.cuda.Stream(device=device))
        self.stage, self.side = streams
        # the first launch on a new stream sets up its hardware queue, which
        # takes milliseconds: do it here rather than in the first step
        for st in (self.stage, self.side):
            with torch.cuda.stream(st):
                torch.zeros(1, device=device)
        self.events = [torch.cuda.Event() for _ in range(2)]
        self.m_ready = torch.cuda.Event()
        for ev in self.events + [self.m_ready]:
            ev.record()  # materialise the HIP events
        # prologue: M_{-1} = stage 1 of q_0, loaded synchronously
        self.dec.select_blocks(q0, cache, block_idx=self.mbuf[2], shape=self.shape)
        torch.cuda.synchronize()
        init = self.mbuf[2].cpu().numpy().astype(np.int32)
        self.ctx = tls_offload_create_ctx(self.shape, host_kv, self.dev_cache, self.maps[0], self.maps[1], init)
        from . import TLS_COPY_DEVICE, TLS_COPY_FULL, tls_offload_get_copy_mode, tls_offload_set_copy_mode
        if copy_mode is not None:
            tls_offload_set_copy_mode(self.ctx, copy_mode)
        self.copy_mode = tls_offload_get_copy_mode(self.ctx)
        self.device_planned = self.copy_mode in (TLS_COPY_DEVICE, TLS_COPY_FULL)
        self.t = 0
        self.copied = []

    @property
    def shape(self):
        """The calls' shape: the current length, strided by the capacity."""
        return shape_of(self.s.with_(N=self.n), self.capacity)

    def selection(self, t):
        """Device buffer holding M_t (valid for three steps after step t)."""
        return self.mbuf[t % 3]

    def append(self, rows):
        """Append rows [B, Hkv, n, row] bf16 (device) to the cache before the
        next step: tls_offload_append on the current stream, after the copies of
        the last prefetch."""
        from . import tls_offload_append
        n = int(rows.shape[2])
        main = torch.cuda.current_stream()
        if self.t > 0:
            main.wait_event(self.events[(self.t - 1) % 2])
        c = self.cache
        tls_offload_append(self.ctx, rows.contiguous(), n, c.label_ch, c.summ, c.codes, c.scale, main)
        self.n += n
        if isinstance(c, GrowingCache):
            c.n = self.n

    def step(self, q_t, helper=None):
        """Enqueue step t; returns the output buffer [B, Hq, DV] (valid after sync).

        Host-planned modes run tls_prefetch_delta on a helper thread (it waits
        for M_t); with device planning it only enqueues, so no thread is used
        unless `helper` is True. `copied` gets |T_t| per step (-1 when the
        device planned it; see total_copied)."""
        import threading
        from . import tls_offload_slot_map, tls_prefetch_delta
        if not self.stagger:
            return self._step_in_order(q_t)
        if helper is None:
            helper = not self.device_planned
        t = self.t
        main = torch.cuda.current_stream()
        mt = self.selection(t)
        sh = self.shape
        self.stage.wait_stream(main)
        with torch.cuda.stream(self.stage):
            self.dec.select_blocks(q_t, self.cache, stream=self.stage, block_idx=mt, shape=sh)
        self.m_ready.record(self.stage)
        self.side.wait_stream(main)
        self.side.wait_event(self.m_ready)
        res = {}

        def prefetch():
            res["n"] = tls_prefetch_delta(self.ctx, t, mt, self.side, self.events[t % 2])

        th = threading.Thread(target=prefetch) if helper else None
        if th:
            th.start()
        else:
            prefetch()
        if t > 0:
            main.wait_event(self.events[(t - 1) % 2])
        self.dec.select_tokens(q_t, self.cache, block_idx=self.selection(t - 1), shape=sh)
        self.dec.decode(q_t, self.dev_cache, slot_map=tls_offload_slot_map(self.ctx, t), slots=self.cap, shape=sh)
        if th:
            th.join()
        self.copied.append(res.get("n", 0))
        self.t += 1
        return self.dec.out

    def _step_in_order(self, q_t):
        from . import tls_offload_slot_map, tls_prefetch_delta
        t = self.t
        main = torch.cuda.current_stream()
        mt = self.selection(t)
        sh = self.shape
        self.dec.select_blocks(q_t, self.cache, block_idx=mt, shape=sh)
        self.copied.append(tls_prefetch_delta(self.ctx, t, mt, main, self.events[t % 2]))
        self.dec.select_tokens(q_t, self.cache, block_idx=mt, shape=sh)
        # the map written by this step's transfer (that of step t+1) holds M_t
        self.dec.decode(q_t, self.dev_cache, slot_map=tls_offload_slot_map(self.ctx, t + 1), slots=self.cap, shape=sh)
        self.t += 1
        return self.dec.out

    def capture(self, queries, outputs=None):
        """Record the next len(queries) steps into a HIP graph and return it
        (a torch.cuda.CUDAGraph; nothing runs until it is replayed).

        Needs planning on the GPU (TLS_COPY_DEVICE or TLS_COPY_FULL): the planning kernel
        keeps its own step count, so the captured launches need no host work.
        `outputs`, if given, is one [B, Hq, DV] fp32 tensor per step that the
        graph fills. The graph holds the buffers of those steps (selections
        rotate over three buffers, slot maps alternate by step parity), so
        replay it once, or repeatedly only when len(queries) is a multiple of 6."""
        if not self.device_planned:
            raise RuntimeError("graph capture needs planning on the GPU (TLS_COPY_DEVICE or TLS_COPY_FULL)")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            main = torch.cuda.current_stream()
            for i, q in enumerate(queries):
                out = self.step(q, helper=False)
                if outputs is not None:
                    outputs[i].copy_(out)
            if self.stagger:
                main.wait_stream(self.stage)
                main.wait_stream(self.side)
        return g

    def last_delta(self):
        from . import tls_offload_last_delta
        counts = np.zeros(self.s.pairs, dtype=np.int32)
        blocks = np.zeros((self.s.pairs, self.kb), dtype=np.int32)
        tls_offload_last_delta(self.ctx, counts, blocks)
        return counts, blocks

    def total_copied(self):
        """Blocks copied since creation over all pairs (synchronises the device)."""
        from . import tls_offload_total_copied
        return tls_offload_total_copied(self.ctx)

    def close(self):
        from . import tls_offload_destroy
        if self.ctx:
            tls_offload_destroy(self.ctx)
            self.ctx = None


class LayeredDecoder:
    """Staggered decode of L layers, each with its own offloaded cache
    (AsyncTLS pages, section 2B, across the layers of a model).

    Layer l of step t runs as one StaggeredDecoder step: its token stage and
    attention on the main stream, after layer l-1's attention (the data
    dependency of a model: layer l's query comes from layer l-1's output);
    its stage 1 for M^l_t on the shared stage stream, which waits for that
    same point; its transfer T^l_t on the shared copy stream. So layer l's
    transfer runs under the attention of the layers after it, and it has until
    layer l of step t+1 -- a whole pass over the other layers -- to land. All
    layers share the two side streams (no more hardware queues than one layer
    uses)."""

    def __init__(self, s, caches, host_kvs, q0s, device="cuda", copy_mode=None, stagger=True):
        streams = (torch.cuda.Stream(device=device), torch.cuda.Stream(device=device))
        for st in streams:
            with torch.cuda.stream(st):
                torch.zeros(1, device=device)
        self.layers = [StaggeredDecoder(s, c, h, q, device, copy_mode, stagger, streams=streams)
                       for c, h, q in zip(caches, host_kvs, q0s)]
        self.stage, self.side = streams

    def step(self, q_layers):
        """Step t of every layer in order; returns the layers' output buffers."""
        return [d.step(q, helper=False) for d, q in zip(self.layers, q_layers)]

    def capture(self, q_steps):
        """One HIP graph of len(q_steps) steps of every layer (q_steps[t][l]);
        planning must be on the GPU (see StaggeredDecoder.capture)."""
        if not all(d.device_planned for d in self.layers):
            raise RuntimeError("graph capture needs planning on the GPU (TLS_COPY_DEVICE or TLS_COPY_FULL)")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            main = torch.cuda.current_stream()
            for qs in q_steps:
                self.step(qs)
            main.wait_stream(self.stage)
            main.wait_stream(self.side)
        return g

    def total_copied(self):
        return sum(d.total_copied() for d in self.layers)

    def close(self):
        for d in self.layers:
            d.close()


def tls_offload_create_ctx(shape, host_kv, dev_cache, map0, map1, init):
    from . import tls_offload_create
    return tls_offload_create(shape, host_kv, dev_cache, map0, map1, init)
