"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
compare each stage with the fp64 oracle.

Selection rule (index sets): with sigma = max |score| over a row's candidates
(oracle scores), scores within 1e-5*sigma of the K-th oracle score form the
band. The GPU set must have the right size, be ascending, contain every
candidate above the band and none below it. Outside the band the sets are
therefore identical; the number of band elements is reported.
Outputs: max-abs error <= 2e-3 against the oracle given identical selections.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workload as W
from two_level_sparse_amd.runtime import Cache, Decoder, bf16

REL_BAND = 1e-5
OUT_TOL = 2e-3


def to_np(t):
    return t.detach().cpu().numpy()


def bf16_bits(t):
    return to_np(t.view(torch.int16)).view(np.uint16)


def unpack_summaries(summ, s, NB=None):
    """The GPU's block summaries (tile-fragment order, see include/tls.h) as
    bf16 bits [pairs, NB, 2, D]: [.., 0, :] Kmax, [.., 1, :] Kmin."""
    bits = bf16_bits(summ).reshape(s.pairs, -1)
    nt = bits.shape[1] // (32 * s.D)
    a = bits.reshape(s.pairs, nt, s.D // 32, 2, 4, 16, 8).transpose(0, 1, 5, 3, 2, 4, 6)
    return a.reshape(s.pairs, nt * 16, 2, s.D)[:, : (s.NB if NB is None else NB)]


def band_check(got, ids, scores, K):
    """Checks a GPU selection `got` (ascending, -1 padded) against oracle scores of
    the candidate ids. Returns (n_band, exact) where exact = same set as the oracle."""
    got = np.asarray(got)
    got = got[got >= 0]
    ids = np.asarray(ids)
    scores = np.asarray(scores, dtype=np.float64)
    k = min(K, ids.size)
    assert got.size == k, (got.size, k)
    assert np.all(np.diff(got) > 0), "selection not ascending/unique"
    sigma = float(np.max(np.abs(scores))) if scores.size else 0.0
    band = REL_BAND * sigma
    order = np.lexsort((ids, -scores))
    sK = scores[order[k - 1]]
    must = set(ids[scores > sK + band].tolist())
    never = set(ids[scores < sK - band].tolist())
    g = set(got.tolist())
    assert must <= g, f"missing {sorted(must - g)[:10]} (above the band)"
    assert not (g & never), f"extra {sorted(g & never)[:10]} (below the band)"
    exact = g == set(ids[order[:k]].tolist())
    n_band = int(np.sum(np.abs(scores - sK) <= band))
    return n_band, exact


class GpuRun:
    """Runs the HIP path for shape s with inputs (q, kv, label_ch) on cuda:0."""

    def __init__(self, s, q, kv, lab):
        self.s = s
        self.q = q
        self.qd = bf16(q)
        self.cache = Cache(s, kv, lab).build()
        self.dec = Decoder(s)
        torch.cuda.synchronize()

    def blocks(self):
        self.dec.select_blocks(self.qd, self.cache, keep_scores=True)
        torch.cuda.synchronize()
        return to_np(self.dec.block_idx).reshape(self.s.pairs, -1), to_np(self.dec.block_score).reshape(self.s.pairs, -1)

    def tokens(self, block_idx=None):
        if block_idx is not None:
            self.dec.block_idx.copy_(torch.from_numpy(np.ascontiguousarray(block_idx, dtype=np.int32))
                                     .reshape(self.dec.block_idx.shape))
        self.dec.select_tokens(self.qd, self.cache)
        torch.cuda.synchronize()
        return to_np(self.dec.token_idx).reshape(self.s.pairs, -1)

    def attend(self, token_idx=None):
        if token_idx is not None:
            self.dec.token_idx.copy_(torch.from_numpy(np.ascontiguousarray(token_idx, dtype=np.int32))
                                     .reshape(self.dec.token_idx.shape))
        self.dec.decode(self.qd, self.cache.kv)
        torch.cuda.synchronize()
        s = self.s
        out = to_np(self.dec.out).reshape(s.B, s.Hkv, s.G, s.DV).reshape(s.pairs, s.G, s.DV)
        lse = to_np(self.dec.lse).reshape(s.pairs, s.G)
        return out, lse


def check_all(s, q, kv, lab, pairs=None, expect_exact=False):
    """Stage-by-stage parity of the HIP path with the oracle on `pairs` (default all).
    Returns a dict of statistics."""
    pairs = np.arange(s.pairs) if pairs is None else np.asarray(pairs)
    run = GpuRun(s, q, kv, lab)
    ref = oracle.decode(s, q, kv, lab, pairs=pairs)
    stats = dict(block_band=0, token_band=0, block_exact=True, token_exact=True)

    # build: summaries, codes and scales bit-exact
    summ = unpack_summaries(run.cache.summ, s)
    codes = to_np(run.cache.codes).reshape(s.pairs, s.N, s.r // 2)
    scale = to_np(run.cache.scale).reshape(s.pairs, s.N)
    for i, p in enumerate(pairs):
        np.testing.assert_array_equal(W.bf16_bits_to_f64(summ[p, :, 0]), ref.kmax[i])
        np.testing.assert_array_equal(W.bf16_bits_to_f64(summ[p, :, 1]), ref.kmin[i])
        np.testing.assert_array_equal(codes[p], oracle.pack_codes(ref.codes[i]))
        np.testing.assert_array_equal(scale[p].view(np.uint32), ref.scale[i].view(np.uint32))

    # stage 1: block scores and sets
    gb, gS = run.blocks()
    kb = min(s.Kb, s.NB)
    for i, p in enumerate(pairs):
        sig = np.max(np.abs(ref.S[i]))
        err = np.max(np.abs(gS[p].astype(np.float64) - ref.S[i]))
        assert err <= REL_BAND * sig, (p, err, sig)
        nb, ex = band_check(gb[p], np.arange(s.NB), ref.S[i], kb)
        stats["block_band"] += nb
        stats["block_exact"] &= ex
        if expect_exact:
            assert ex and gb[p].tolist() == ref.block_idx[i].tolist()

    # stage 2 on the oracle's block sets
    forced_blocks = gb.copy()
    forced_blocks[pairs] = ref.block_idx
    gt = run.tokens(forced_blocks)
    for i, p in enumerate(pairs):
        b, h = divmod(int(p), s.Hkv)
        qp = q[b, h * s.G:(h + 1) * s.G]
        tok, cand, cs = oracle.select_tokens_pair(s, qp, lab[h], ref.codes[i], ref.scale[i], ref.block_idx[i])
        nb, ex = band_check(gt[p], cand, cs, s.Kt)
        stats["token_band"] += nb
        stats["token_exact"] &= ex
        if expect_exact:
            assert ex

    # attention on the oracle's token sets
    kt = min(s.Kt, kb * s.bs)
    forced_tokens = gt.copy()
    for i, p in enumerate(pairs):
        forced_tokens[p] = -1
        forced_tokens[p, : ref.ntok[i]] = ref.token_idx[i, : ref.ntok[i]]
    out, lse = run.attend(forced_tokens)
    err = max(np.max(np.abs(out[p] - ref.out[i])) for i, p in enumerate(pairs))
    lerr = max(np.max(np.abs(lse[p] - ref.lse[i])) for i, p in enumerate(pairs))
    assert err <= OUT_TOL, err
    assert lerr <= OUT_TOL, lerr
    stats["out_err"] = float(err)
    stats["lse_err"] = float(lerr)

    # the whole chain on the GPU's own selections
    run.dec.select_blocks(run.qd, run.cache)
    run.dec.select_tokens(run.qd, run.cache)
    out2, lse2 = run.attend()
    gt2 = to_np(run.dec.token_idx).reshape(s.pairs, -1)
    chain_err = 0.0
    for i, p in enumerate(pairs):
        b, h = divmod(int(p), s.Hkv)
        tk = gt2[p][gt2[p] >= 0]
        o_ref, l_ref = oracle.attend_pair(s, q[b, h * s.G:(h + 1) * s.G], kv[b, h], tk)
        chain_err = max(chain_err, float(np.max(np.abs(out2[p] - o_ref))))
    assert chain_err <= OUT_TOL, chain_err
    stats["chain_err"] = chain_err

    # both stages in one call (tls_select, the path the benchmark times): the
    # same sets as the two calls, and each checked against the oracle on its
    # own -- blocks by the band rule on the oracle's block scores, tokens by the
    # band rule on the oracle's candidate scores over the call's own block set
    bi_sep = to_np(run.dec.block_idx).copy()
    run.dec.block_idx.fill_(-7)
    run.dec.token_idx.fill_(-7)
    run.dec.select(run.qd, run.cache)
    torch.cuda.synchronize()
    bi_sel = to_np(run.dec.block_idx).reshape(s.pairs, -1)
    ti_sel = to_np(run.dec.token_idx).reshape(s.pairs, -1)
    np.testing.assert_array_equal(bi_sel.reshape(bi_sep.shape), bi_sep)
    np.testing.assert_array_equal(ti_sel, gt2)
    for i, p in enumerate(pairs):
        b, h = divmod(int(p), s.Hkv)
        band_check(bi_sel[p], np.arange(s.NB), ref.S[i], kb)
        _, cand, cs = oracle.select_tokens_pair(s, q[b, h * s.G:(h + 1) * s.G], lab[h], ref.codes[i],
                                                ref.scale[i], bi_sel[p])
        band_check(ti_sel[p], cand, cs, s.Kt)
    stats["kt"] = kt

    # the whole step in one launch (tls_decode_step, where it covers the shape):
    # the same sets as tls_select (the same arithmetic), outputs within 2e-3 of
    # the oracle's attention over its own token sets; twice in a row, since
    # the launch must leave its workspace ready for the next one
    if run.dec.one_launch:
        out_sep = to_np(run.dec.out).copy()
        for rep in range(2):
            run.dec.block_idx.fill_(-7)
            run.dec.token_idx.fill_(-7)
            run.dec.out.fill_(float("nan"))
            run.dec.step_one_launch(run.qd, run.cache)
            run.dec.step_status()
            bi1 = to_np(run.dec.block_idx).reshape(s.pairs, -1)
            ti1 = to_np(run.dec.token_idx).reshape(s.pairs, -1)
            np.testing.assert_array_equal(bi1, bi_sel)
            np.testing.assert_array_equal(ti1, ti_sel)
            o1 = to_np(run.dec.out).reshape(s.pairs, s.G, s.DV)
            l1 = to_np(run.dec.lse).reshape(s.pairs, s.G)
            step_err = 0.0
            for i, p in enumerate(pairs):
                b, h = divmod(int(p), s.Hkv)
                tk = ti1[p][ti1[p] >= 0]
                o_ref, l_ref = oracle.attend_pair(s, q[b, h * s.G:(h + 1) * s.G], kv[b, h], tk)
                step_err = max(step_err, float(np.max(np.abs(o1[p] - o_ref))), float(np.max(np.abs(l1[p] - l_ref))))
            assert step_err <= OUT_TOL, step_err
            # every pair, checked or not, agrees with the separate calls' attention
            sep = out_sep.reshape(s.pairs, s.G, s.DV)
            assert float(np.max(np.abs(o1 - sep))) <= 1e-4
        stats["one_launch_err"] = step_err
    return stats
