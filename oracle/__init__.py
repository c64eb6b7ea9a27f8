"""fp64 CPU oracle for the two-level sparse-attention decode step (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP path in
``two_level_sparse_amd``; the two meet only in ``workload`` (seeded inputs).

The arithmetic lives in ``tls_oracle.c`` (plain C, double precision, OpenMP
over (batch, kv-head) pairs); this module builds it with gcc and wraps it with
ctypes and numpy. Every function follows the AsyncTLS pages, section 2
"Methodology"; the C file documents each step and the readings taken where
the pages are silent.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "tls_oracle.c"
_LIB = _HERE / "liboracle.so"


def build(force: bool = True) -> Path:
    """Compile liboracle.so with gcc (-O2, OpenMP, IEEE double: no fast-math)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", "-o", str(tmp), str(_SRC), "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Shape(C.Structure):
    _fields_ = [("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("D", C.c_int32),
                ("DV", C.c_int32), ("row", C.c_int32), ("v_off", C.c_int32), ("N", C.c_int64),
                ("bs", C.c_int32), ("r", C.c_int32), ("Kb", C.c_int32), ("Kt", C.c_int32),
                ("sm_scale", C.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        _lib = C.CDLL(str(_LIB))
    return _lib


def _shape(s) -> _Shape:
    return _Shape(s.B, s.Hq, s.Hkv, s.D, s.DV, s.row, s.v_off, s.N, s.bs, s.r, s.Kb, s.Kt,
                  float(s.sm_scale))


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def topk(scores, K, ids=None):
    """Top-K by (score desc, index asc), returned ascending (lower index wins ties)."""
    scores = _c(scores, np.float64)
    ids = None if ids is None else _c(ids, np.int32)
    out = np.empty(max(0, min(int(K), scores.size)), dtype=np.int32)
    n = lib().orc_topk(_p(scores), _p(ids), C.c_int64(scores.size), C.c_int64(int(K)), _p(out))
    assert n == out.size, n
    return out


def summaries_pair(s, kv_pair):
    """Per-block key max and min of one pair: ([NB, D], [NB, D]) float64."""
    kv_pair = _c(kv_pair, np.uint16)
    kmax = np.empty((s.NB, s.D)); kmin = np.empty((s.NB, s.D))
    sh = _shape(s)
    lib().orc_summaries_pair(C.byref(sh), _p(kv_pair), _p(kmax), _p(kmin))
    return kmax, kmin


def quantize_pair(s, kv_pair, lab):
    """INT4 label cache of one pair: (codes [N, r] int8, scale [N] float32)."""
    kv_pair = _c(kv_pair, np.uint16); lab = _c(lab, np.int32)
    codes = np.empty((s.N, s.r), dtype=np.int8); scale = np.empty(s.N, dtype=np.float32)
    sh = _shape(s)
    lib().orc_quantize_pair(C.byref(sh), _p(kv_pair), _p(lab), _p(codes), _p(scale))
    return codes, scale


def pack_codes(codes):
    codes = _c(codes, np.int8)
    n, r = codes.shape
    out = np.empty((n, r // 2), dtype=np.uint8)
    lib().orc_pack_codes(_p(codes), C.c_int64(n), C.c_int(r), _p(out))
    return out


def select_blocks_pair(s, q_pair, kmax, kmin):
    """Stage 1 for one pair: (block_idx ascending, S [NB], s_head [G, NB])."""
    q_pair = _c(q_pair, np.uint16); kmax = _c(kmax, np.float64); kmin = _c(kmin, np.float64)
    s_head = np.empty((s.G, s.NB)); S = np.empty(s.NB)
    idx = np.empty(min(s.Kb, s.NB), dtype=np.int32)
    sh = _shape(s)
    n = lib().orc_select_blocks_pair(C.byref(sh), _p(q_pair), _p(kmax), _p(kmin), _p(s_head), _p(S), _p(idx))
    if n < 0:
        raise RuntimeError(f"oracle block stage failed ({n})")
    return idx[:n], S, s_head


def select_tokens_pair(s, q_pair, lab, codes, scale, block_idx):
    """Stage 2 for one pair: (token_idx ascending, candidate tokens, candidate scores)."""
    q_pair = _c(q_pair, np.uint16); lab = _c(lab, np.int32); codes = _c(codes, np.int8)
    scale = _c(scale, np.float32); block_idx = _c(block_idx, np.int32)
    cap = max(1, block_idx.size * s.bs)
    tok = np.empty(max(1, min(s.Kt, cap)), dtype=np.int32)
    cand = np.empty(cap, dtype=np.int32); cs = np.empty(cap)
    nc = C.c_int64(0)
    sh = _shape(s)
    n = lib().orc_select_tokens_pair(C.byref(sh), _p(q_pair), _p(lab), _p(codes), _p(scale), _p(block_idx),
                                     C.c_int(block_idx.size), _p(tok), _p(cand), _p(cs), C.byref(nc))
    if n < 0:
        raise RuntimeError("oracle token stage failed")
    return tok[:n], cand[: nc.value], cs[: nc.value]


def attend_pair(s, q_pair, kv_pair, tok):
    """Exact attention of the G heads over the tokens `tok`: (out [G, DV], lse [G])."""
    q_pair = _c(q_pair, np.uint16); kv_pair = _c(kv_pair, np.uint16); tok = _c(tok, np.int32)
    out = np.empty((s.G, s.DV)); lse = np.empty(s.G)
    sh = _shape(s)
    lib().orc_attend_pair(C.byref(sh), _p(q_pair), _p(kv_pair), _p(tok), C.c_int(tok.size), _p(out), _p(lse))
    return out, lse


class Step:
    """Results of one decode step for a list of pairs (index 0 .. len(pairs)-1)."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def decode(s, q, kv, label_ch, pairs=None, built=None, force_blocks=None, force_tokens=None):
    """Full decode step (O1..O9) for `pairs` (default: all) of shape `s`.

    q [B, Hq, D] and kv [B, Hkv, N, row] are bf16 bit arrays. `built` may pass a
    previous Step to reuse its summaries and label cache. `force_blocks` /
    `force_tokens` ([np, Kb'] / list of arrays) replace the selections of the
    earlier stages, so each stage can be compared on identical inputs.
    """
    pairs = np.arange(s.pairs, dtype=np.int32) if pairs is None else _c(pairs, np.int32)
    np_ = pairs.size
    q = _c(q, np.uint16); kv = _c(kv, np.uint16); label_ch = _c(label_ch, np.int32)
    kb = min(s.Kb, s.NB)
    kt = min(s.Kt, kb * s.bs)
    if built is None:
        kmax = np.empty((np_, s.NB, s.D)); kmin = np.empty((np_, s.NB, s.D))
        codes = np.empty((np_, s.N, s.r), dtype=np.int8); scale = np.empty((np_, s.N), dtype=np.float32)
        build_flag = 1
    else:
        kmax, kmin, codes, scale = built.kmax, built.kmin, built.codes, built.scale
        build_flag = 0
    fb = None if force_blocks is None else _c(force_blocks, np.int32).reshape(np_, kb)
    ft = fn = None
    if force_tokens is not None:
        ft = np.zeros((np_, kt), dtype=np.int32); fn = np.zeros(np_, dtype=np.int32)
        for i, t in enumerate(force_tokens):
            t = np.asarray(t, dtype=np.int32); t = t[t >= 0]
            ft[i, : t.size] = t; fn[i] = t.size
    S = np.empty((np_, s.NB)); bi = np.empty((np_, kb), dtype=np.int32)
    ti = np.full((np_, kt), -1, dtype=np.int32); nt = np.empty(np_, dtype=np.int32)
    out = np.empty((np_, s.G, s.DV)); lse = np.empty((np_, s.G))
    sh = _shape(s)
    rc = lib().orc_decode(C.byref(sh), _p(q), _p(kv), _p(label_ch), _p(pairs), C.c_int(np_), C.c_int(build_flag),
                          _p(kmax), _p(kmin), _p(codes), _p(scale), _p(fb), _p(ft), _p(fn),
                          _p(S), _p(bi), _p(ti), _p(nt), _p(out), _p(lse))
    if rc != 0:
        raise RuntimeError(f"oracle decode failed ({rc})")
    return Step(pairs=pairs, kmax=kmax, kmin=kmin, codes=codes, scale=scale, S=S, block_idx=bi,
                token_idx=ti, ntok=nt, out=out, lse=lse)


def staggered(s, qs, kv, label_ch, built, force_prologue=None, force_M=None, lens=None):
    """Staggered offloaded schedule (O10) over all pairs; `built` = decode(...) over all pairs.

    force_prologue [np, Kb'] / force_M [steps, np, Kb'] replace the schedule's own
    block selections (the prologue's and each step's), so that a run whose sets
    differ only inside the score band can be followed step by step.
    lens [steps + 1]: a cache that grows between steps (s.N = the allocated
    length, kv holding all of it): the prologue sees lens[0] tokens, step t
    lens[t + 1]; built's codes and scales (of all s.N tokens) are used, its
    summaries are not (the schedule builds them from each prefix)."""
    steps = qs.shape[0]
    qs = _c(qs, np.uint16); kv = _c(kv, np.uint16); label_ch = _c(label_ch, np.int32)
    np_ = s.pairs
    kb = min(s.Kb, s.NB)
    M = np.empty((steps, np_, kb), dtype=np.int32); T = np.full((steps, np_, kb), -1, dtype=np.int32)
    nT = np.empty((steps, np_), dtype=np.int32); ne = np.empty((steps, np_), dtype=np.int32)
    ev = np.full((steps, np_, 2 * kb), -1, dtype=np.int32)
    out = np.empty((steps, np_, s.G, s.DV)); lse = np.empty((steps, np_, s.G))
    sh = _shape(s)
    rc = lib().orc_staggered(C.byref(sh), C.c_int(steps), _p(qs), _p(kv), _p(label_ch),
                             _p(_c(built.kmax, np.float64)), _p(_c(built.kmin, np.float64)),
                             _p(_c(built.codes, np.int8)), _p(_c(built.scale, np.float32)),
                             _p(None if force_prologue is None else _c(force_prologue, np.int32)),
                             _p(None if force_M is None else _c(force_M, np.int32)),
                             _p(None if lens is None else _c(lens, np.int64)),
                             _p(M), _p(T), _p(nT), _p(ne), _p(ev), _p(out), _p(lse))
    if rc != 0:
        raise RuntimeError(f"oracle staggered schedule failed ({rc})")
    return Step(M=M, T=T, nT=nT, nevict=ne, evicted=ev, out=out, lse=lse)
