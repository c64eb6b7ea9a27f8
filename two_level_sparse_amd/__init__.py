"""two_level_sparse_amd -- MI355X (gfx950) two-level sparse-attention decode.

Thin ctypes binding over libtls.so (the C ABI declared in include/tls.h). The
functions here carry the C names and only marshal arguments: every step of
the decode path runs in the HIP kernels of the library. PyTorch is used for
device memory and streams only. If libtls.so has not been built the import
of the binding fails loudly; there is no CPU fallback.

Method: AsyncTLS two-level sparse attention (pages "AsyncTLS: Efficient
Generative LLM Inference with Asynchronous Two-level Sparse Attention",
section 2): block filtering by a Quest bound computed as a GEMM, token
selection on INT4 label channels, attention over the kept tokens, and a
staggered incremental prefetch of offloaded KV blocks.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libtls.so"

TLS_OK = 0
TLS_ERR_INVALID_ARG = -1
TLS_ERR_UNSUPPORTED = -2
TLS_ERR_WORKSPACE = -3
TLS_ERR_HIP = -4
TLS_ERR_STATE = -5
TLS_WS_BLOCKS, TLS_WS_TOKENS, TLS_WS_DECODE, TLS_WS_SELECT, TLS_WS_STEP = 0, 1, 2, 3, 4

TLS_COPY_GATHER, TLS_COPY_MEMCPY, TLS_COPY_DEVICE, TLS_COPY_FULL = 0, 1, 2, 3
TLS_PROFILE_BLOCK_SCORES, TLS_PROFILE_ATTENTION, TLS_PROFILE_HOST_COPY = 0, 1, 2
TLS_NOALLOC_SCRATCH_BYTES = 40 << 20  # the device array of tls_sparse_decode_noalloc

EXPORTED = ["tls_workspace_size", "tls_build_summaries", "tls_select_blocks", "tls_select_tokens", "tls_select",
            "tls_sparse_decode", "tls_sparse_decode_noalloc", "tls_decode_step", "tls_decode_step_status", "tls_append_kv", "tls_offload_create", "tls_offload_slot_map", "tls_prefetch_delta",
            "tls_offload_set_copy_mode", "tls_offload_append", "tls_offload_get_copy_mode", "tls_offload_last_delta",
            "tls_offload_total_copied", "tls_offload_destroy", "tls_profile_events",
            "tls_last_error", "tls_version"]


class tls_shape_t(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim_qk", C.c_int32), ("head_dim_v", C.c_int32), ("v_is_k_prefix", C.c_int32),
                ("ctx_len", C.c_int64), ("block_size", C.c_int32), ("num_label_ch", C.c_int32),
                ("top_kb", C.c_int32), ("top_kt", C.c_int32), ("sm_scale", C.c_float),
                ("ctx_capacity", C.c_int64)]


class TlsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None


def load_library(path: Path | str | None = None) -> C.CDLL:
    """Load libtls.so (built in-tree by two_level_sparse_amd/build.py)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise ImportError(f"{p} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python two_level_sparse_amd/build.py`")
    lib = C.CDLL(str(p))
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sh = C.POINTER(tls_shape_t)
    sig = {
        "tls_workspace_size": (sz, [sh, C.c_int]),
        "tls_build_summaries": (C.c_int, [sh, vp, vp, vp, vp, vp, vp]),
        "tls_append_kv": (C.c_int, [sh, vp, i32, vp, vp, vp, vp, vp, vp]),
        "tls_select_blocks": (C.c_int, [sh, vp, vp, vp, vp, vp, sz, vp]),
        "tls_select_tokens": (C.c_int, [sh, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "tls_select": (C.c_int, [sh, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "tls_sparse_decode": (C.c_int, [sh, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]),
        "tls_sparse_decode_noalloc": (C.c_int, [sh, vp, vp, vp, i32, vp, vp, vp, vp]),
        "tls_decode_step": (C.c_int, [sh, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "tls_decode_step_status": (C.c_int, [vp, vp]),
        "tls_offload_create": (C.c_int, [sh, vp, vp, vp, vp, vp, C.POINTER(vp)]),
        "tls_offload_slot_map": (vp, [vp, i32]),
        "tls_prefetch_delta": (C.c_int, [vp, i32, vp, vp, vp, C.POINTER(i64)]),
        "tls_offload_last_delta": (C.c_int, [vp, vp, vp]),
        "tls_offload_append": (C.c_int, [vp, vp, i32, vp, vp, vp, vp, vp]),
        "tls_offload_set_copy_mode": (C.c_int, [vp, C.c_int]),
        "tls_offload_get_copy_mode": (C.c_int, [vp]),
        "tls_offload_total_copied": (C.c_int, [vp, C.POINTER(i64)]),
        "tls_offload_destroy": (None, [vp]),
        "tls_profile_events": (C.c_int, [C.c_int, vp, vp]),
        "tls_last_error": (C.c_char_p, []),
        "tls_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(rc):
    if rc != TLS_OK:
        raise TlsError(rc, load_library().tls_last_error().decode())


def _ptr(t):
    """Device (or host) address of a torch tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def shape_of(s, capacity: int = 0) -> tls_shape_t:
    """tls_shape_t from any object with the workload attributes (B, Hq, Hkv, D, DV, ...);
    `capacity`: allocated tokens per sequence (0: exactly N)."""
    return tls_shape_t(s.B, s.Hq, s.Hkv, s.D, s.DV, int(bool(s.v_is_k_prefix)), s.N, s.bs, s.r, s.Kb, s.Kt,
                       float(s.sm_scale), int(capacity))


def tls_workspace_size(shape: tls_shape_t, which: int) -> int:
    return int(load_library().tls_workspace_size(C.byref(shape), which))


def tls_build_summaries(shape, kv, label_ch, summ, codes, scale, stream=None):
    _check(load_library().tls_build_summaries(C.byref(shape), _ptr(kv), _ptr(label_ch), _ptr(summ), _ptr(codes),
                                              _ptr(scale), _stream(stream)))


def tls_append_kv(shape, new_kv, n_new, kv, label_ch, summ, codes, scale, stream=None):
    """shape.ctx_len: the length before the append; shape.ctx_capacity: the allocated length."""
    _check(load_library().tls_append_kv(C.byref(shape), _ptr(new_kv), int(n_new), _ptr(kv), _ptr(label_ch),
                                        _ptr(summ), _ptr(codes), _ptr(scale), _stream(stream)))


def tls_select_blocks(shape, q, summ, block_idx, block_score=None, ws=None, ws_bytes=0, stream=None):
    _check(load_library().tls_select_blocks(C.byref(shape), _ptr(q), _ptr(summ), _ptr(block_idx), _ptr(block_score),
                                            _ptr(ws), ws_bytes, _stream(stream)))


def tls_select_tokens(shape, q, label_ch, codes, scale, block_idx, token_idx, ws=None, ws_bytes=0, stream=None):
    _check(load_library().tls_select_tokens(C.byref(shape), _ptr(q), _ptr(label_ch), _ptr(codes), _ptr(scale),
                                            _ptr(block_idx), _ptr(token_idx), _ptr(ws), ws_bytes, _stream(stream)))


def tls_select(shape, q, summ, label_ch, codes, scale, block_idx, token_idx, ws=None, ws_bytes=0, stream=None):
    _check(load_library().tls_select(C.byref(shape), _ptr(q), _ptr(summ), _ptr(label_ch), _ptr(codes), _ptr(scale),
                                     _ptr(block_idx), _ptr(token_idx), _ptr(ws), ws_bytes, _stream(stream)))


def tls_sparse_decode(shape, q, kv_cache, slot_map, slots_per_pair, token_idx, out, lse=None, ws=None, ws_bytes=0,
                      stream=None):
    _check(load_library().tls_sparse_decode(C.byref(shape), _ptr(q), _ptr(kv_cache), _ptr(slot_map),
                                            int(slots_per_pair), _ptr(token_idx), _ptr(out), _ptr(lse), _ptr(ws),
                                            ws_bytes, _stream(stream)))


def tls_sparse_decode_noalloc(shape, q, kv_cache, slot_map, slots_per_pair, token_idx, out, lse=None, stream=None):
    """tls_sparse_decode with the split partials in the library's own device
    array (no workspace; calls on one GPU must not overlap)."""
    _check(load_library().tls_sparse_decode_noalloc(C.byref(shape), _ptr(q), _ptr(kv_cache), _ptr(slot_map),
                                                    int(slots_per_pair), _ptr(token_idx), _ptr(out), _ptr(lse),
                                                    _stream(stream)))


def tls_decode_step(shape, q, summ, label_ch, codes, scale, kv, block_idx, token_idx, out, lse=None, ws=None,
                    ws_bytes=0, stream=None):
    """Both selection stages and the attention in one launch; ws must be
    zero-filled before its first use (every call leaves it so)."""
    _check(load_library().tls_decode_step(C.byref(shape), _ptr(q), _ptr(summ), _ptr(label_ch), _ptr(codes),
                                          _ptr(scale), _ptr(kv), _ptr(block_idx), _ptr(token_idx), _ptr(out),
                                          _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def tls_decode_step_status(ws, stream=None):
    _check(load_library().tls_decode_step_status(_ptr(ws), _stream(stream)))


def tls_offload_create(shape, host_kv, dev_cache, slot_map0, slot_map1, initial_blocks):
    """Returns an opaque context handle (int). `initial_blocks` is a host int32 tensor/array."""
    h = C.c_void_p()
    init = initial_blocks.ctypes.data if hasattr(initial_blocks, "ctypes") else _ptr(initial_blocks)
    _check(load_library().tls_offload_create(C.byref(shape), _ptr(host_kv), _ptr(dev_cache), _ptr(slot_map0),
                                             _ptr(slot_map1), init, C.byref(h)))
    return h.value


def tls_offload_slot_map(ctx, step) -> int:
    return load_library().tls_offload_slot_map(ctx, step)


def tls_prefetch_delta(ctx, step, dev_block_idx, side_stream, copies_done_event) -> int:
    n = C.c_int64(0)
    _check(load_library().tls_prefetch_delta(ctx, step, _ptr(dev_block_idx), _stream(side_stream),
                                             copies_done_event.cuda_event, C.byref(n)))
    return n.value


def tls_offload_append(ctx, new_kv, n_new, label_ch, summ, codes, scale, stream=None):
    _check(load_library().tls_offload_append(ctx, _ptr(new_kv), int(n_new), _ptr(label_ch), _ptr(summ), _ptr(codes),
                                             _ptr(scale), _stream(stream)))


def tls_offload_set_copy_mode(ctx, mode):
    _check(load_library().tls_offload_set_copy_mode(ctx, int(mode)))


def tls_offload_get_copy_mode(ctx) -> int:
    rc = load_library().tls_offload_get_copy_mode(ctx)
    if rc < 0:
        _check(rc)
    return rc


def tls_offload_total_copied(ctx) -> int:
    n = C.c_int64(0)
    _check(load_library().tls_offload_total_copied(ctx, C.byref(n)))
    return n.value


def tls_offload_last_delta(ctx, counts, blocks):
    """counts / blocks: host numpy int32 arrays [pairs] and [pairs, Kb']."""
    _check(load_library().tls_offload_last_delta(ctx, counts.ctypes.data, blocks.ctypes.data))


def tls_offload_destroy(ctx):
    load_library().tls_offload_destroy(ctx)


def tls_profile_events(which, start_event=None, end_event=None):
    """torch.cuda.Event pair recorded around kernel `which` (TLS_PROFILE_*) of
    every later call that launches it (None, None: off). A torch event gets its
    HIP handle at its first record, so unrecorded events are recorded once here
    (the library's later record replaces that timestamp)."""
    handles = []
    for ev in (start_event, end_event):
        if ev is None:
            handles.append(None)
            continue
        if not ev.cuda_event:
            ev.record()
        handles.append(ev.cuda_event)
    _check(load_library().tls_profile_events(int(which), handles[0], handles[1]))


def tls_version() -> str:
    return load_library().tls_version().decode()
