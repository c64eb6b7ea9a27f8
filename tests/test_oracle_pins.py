"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the property it checks. The method is the one on the AsyncTLS
pages, section 2 "Methodology"; the pages print no numbers, so the pins are a
hand-worked example, closed forms, special cases that reduce to library
routines (numpy top-k on exact dot products, torch's dense attention in
float64, scipy's logsumexp), brute force on tiny inputs, and invariants.
"""
import itertools
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
import workload as W

GOLD = Path(__file__).resolve().parent / "golden"


def bits(x):
    """float values that are exact in bf16 -> bf16 bit patterns (checked exact)."""
    x = np.asarray(x, dtype=np.float32)
    b = W.f32_to_bf16_bits(x)
    assert np.array_equal(W.bf16_bits_to_f32(b), x), "value not representable in bf16"
    return b


def f64(b):
    return W.bf16_bits_to_f64(b)


def make_inputs(s, rng, int_range=None):
    """Random q [B,Hq,D] and kv [B,Hkv,N,row] for shape s; integer-valued if int_range."""
    if int_range is None:
        q = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
        kv = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32))
    else:
        q = bits(rng.integers(-int_range, int_range + 1, (s.B, s.Hq, s.D)))
        kv = bits(rng.integers(-int_range, int_range + 1, (s.B, s.Hkv, s.N, s.row)))
    return q, kv


def lab_all(s):
    return np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))


def rank_desc(scores):
    """numpy top order: score desc, index asc."""
    return np.lexsort((np.arange(scores.size), -scores))


# ---------------------------------------------------------------- golden --

def test_hand_worked_example():
    """The hand-derived 6-token case of tests/golden (every intermediate value)."""
    ex = json.loads((GOLD / "hand_worked_example.json").read_text())
    s = W.small_shape(B=1, Hq=2, Hkv=1, D=2, DV=2, N=6, bs=2, r=2, Kb=2, Kt=2, n_outlier=0).with_(sm=1.0)
    k = np.array(ex["k"], dtype=np.float32); v = np.array(ex["v"], dtype=np.float32)
    kv = bits(np.concatenate([k, v], axis=1))
    q = bits(np.array(ex["q"], dtype=np.float32))
    lab = np.array(ex["label_ch"], dtype=np.int32)
    kmax, kmin = oracle.summaries_pair(s, kv)
    assert np.array_equal(kmax, ex["kmax"]) and np.array_equal(kmin, ex["kmin"])
    bi, S, s_head = oracle.select_blocks_pair(s, q, kmax, kmin)
    assert np.array_equal(s_head, ex["s_head"]) and np.array_equal(S, ex["S"])
    assert bi.tolist() == ex["block_idx"]
    codes, scale = oracle.quantize_pair(s, kv, lab)
    assert codes[:4].tolist() == ex["codes"]
    f17, f27 = float(np.float32(1 / 7)), float(np.float32(2 / 7))
    assert scale[:4].tolist() == [f17, f17, f27, f27]
    tok, cand, cs = oracle.select_tokens_pair(s, q, lab, codes, scale, bi)
    assert cand.tolist() == [0, 1, 2, 3]
    assert cs.tolist() == [7 * f17, 3.5 * f17, 13 * f27, 14 * f27]
    assert tok.tolist() == ex["token_idx"]
    out, lse = oracle.attend_pair(s, q, kv, tok)
    np.testing.assert_allclose(out, ex["out"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, ex["lse"], rtol=0, atol=1e-15)


# --------------------------------------------------------------- top-k ----

def test_topk_brute_force_with_ties():
    """The oracle's top-k is the unique set dominating every outside element under
    (score desc, index asc); every size-K subset is enumerated (integer scores force ties)."""
    rng = np.random.default_rng(0)
    for trial in range(30):
        n = int(rng.integers(1, 13)); K = int(rng.integers(1, n + 2))
        sc = rng.integers(-3, 4, n).astype(np.float64)
        got = oracle.topk(sc, K)
        k = min(K, n)
        winners = []
        for sub in itertools.combinations(range(n), k):
            inside = set(sub)
            ok = all((sc[i] > sc[j]) or (sc[i] == sc[j] and i < j)
                     for i in inside for j in range(n) if j not in inside)
            if ok:
                winners.append(sub)
        assert len(winners) == 1
        assert got.tolist() == list(winners[0])


# ----------------------------------------------------------- summaries ----

@pytest.mark.parametrize("N,bs", [(1000, 64), (256, 16), (64, 64), (5, 4)])
def test_summaries_match_numpy_block_reduce(N, bs):
    s = W.small_shape(N=N, bs=bs, B=1, Hkv=1, Hq=2, D=32, DV=16)
    rng = np.random.default_rng(N)
    _, kv = make_inputs(s, rng)
    kmax, kmin = oracle.summaries_pair(s, kv[0, 0])
    k = f64(kv[0, 0, :, : s.D])
    pad = s.NB * bs - N
    kp = np.concatenate([k, np.full((pad, s.D), np.nan)]) if pad else k
    kp = kp.reshape(s.NB, bs, s.D)
    np.testing.assert_array_equal(kmax, np.nanmax(kp, axis=1))
    np.testing.assert_array_equal(kmin, np.nanmin(kp, axis=1))


# ---------------------------------------------------------- block stage ----

@pytest.mark.parametrize("G", [1, 4, 8])
def test_block_score_is_upper_bound(G):
    """Every q_g . k_t with t in block j is <= s[g,j], and S[j] >= all of them."""
    s = W.small_shape(B=1, Hq=G, Hkv=1, N=700, bs=32, D=64, DV=64, Kb=5)
    rng = np.random.default_rng(G)
    q, kv = make_inputs(s, rng)
    kmax, kmin = oracle.summaries_pair(s, kv[0, 0])
    bi, S, s_head = oracle.select_blocks_pair(s, q[0], kmax, kmin)
    qq = f64(q[0]); kk = f64(kv[0, 0, :, : s.D])
    dots = qq @ kk.T                        # [G, N] exact products, float64 sums
    mag = np.abs(qq) @ np.abs(kk).T
    blk = np.arange(s.N) // s.bs
    assert np.all(s_head[:, blk] >= dots - 1e-12 * mag)
    assert np.all(S[blk] >= dots.max(axis=0) - 1e-12 * mag.max(axis=0))
    np.testing.assert_array_equal(S, s_head.max(axis=0))


def test_block_size_one_is_exact_topk_of_dot_products():
    """bs = 1: Kmax = Kmin = k, so S = max_g q_g.k exactly and stage 1 is exact top-k."""
    s = W.small_shape(B=1, Hq=4, Hkv=1, N=300, bs=1, D=32, DV=32, Kb=17)
    rng = np.random.default_rng(3)
    q, kv = make_inputs(s, rng, int_range=3)   # integer data: exact sums and many ties
    kmax, kmin = oracle.summaries_pair(s, kv[0, 0])
    bi, S, _ = oracle.select_blocks_pair(s, q[0], kmax, kmin)
    dots = (f64(q[0]) @ f64(kv[0, 0, :, : s.D]).T).max(axis=0)
    np.testing.assert_array_equal(S, dots)
    assert bi.tolist() == sorted(rank_desc(dots)[: s.Kb].tolist())


def test_block_selection_brute_force_tiny():
    """N=256, bs=16, NB=16, Kb=4, d=8, G=2: all C(16,4) subsets are enumerated."""
    s = W.small_shape(B=1, Hq=2, Hkv=1, N=256, bs=16, D=8, DV=8, r=4, Kb=4, Kt=16)
    rng = np.random.default_rng(11)
    for trial in range(5):
        q, kv = make_inputs(s, rng, int_range=1)
        kmax, kmin = oracle.summaries_pair(s, kv[0, 0])
        bi, S, _ = oracle.select_blocks_pair(s, q[0], kmax, kmin)
        wins = [sub for sub in itertools.combinations(range(16), 4)
                if all((S[i] > S[j]) or (S[i] == S[j] and i < j) for i in sub for j in range(16) if j not in sub)]
        assert len(wins) == 1 and list(wins[0]) == bi.tolist()


# ------------------------------------------------------------ quantizer ----

def test_quantizer_bounds_and_grid_round_trip():
    s = W.small_shape(B=1, Hq=2, Hkv=1, N=2000, bs=64, D=64, DV=64, r=16)
    rng = np.random.default_rng(5)
    _, kv = make_inputs(s, rng)
    lab = np.sort(rng.choice(s.D, s.r, replace=False)).astype(np.int32)
    codes, scale = oracle.quantize_pair(s, kv[0, 0], lab)
    k = f64(kv[0, 0][:, lab])
    assert codes.min() >= -7 and codes.max() <= 7
    assert np.all(np.abs(codes * scale.astype(np.float64)[:, None] - k) <= scale[:, None] * 0.5 * (1 + 1e-6))
    # the channel of largest magnitude maps to +-7
    amax = np.abs(k).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(s.N), amax]) == 7)
    np.testing.assert_array_equal(scale, (np.abs(k).max(axis=1) / 7.0).astype(np.float32))

    # grid-aligned keys k = m * 2^e with max |m| = 7 round-trip exactly
    m = rng.integers(-7, 8, (s.N, s.r)); m[:, 0] = 7 * np.where(rng.random(s.N) < 0.5, 1, -1)
    e = rng.integers(-3, 3, (s.N, 1)).astype(np.float64)
    kg = (m * 2.0 ** e).astype(np.float32)
    kv2 = np.zeros((s.N, s.row), dtype=np.uint16)
    kv2[:, lab] = bits(kg)
    codes2, scale2 = oracle.quantize_pair(s, kv2, lab)
    np.testing.assert_array_equal(codes2, m)
    np.testing.assert_array_equal(codes2 * scale2.astype(np.float64)[:, None], kg)


def test_quantizer_zero_token_and_packing():
    s = W.small_shape(B=1, Hq=2, Hkv=1, N=3, bs=4, D=8, DV=8, r=4)
    lab = np.array([0, 2, 5, 7], dtype=np.int32)
    kv = np.zeros((3, s.row), dtype=np.uint16)
    kv[1, lab] = bits([-7.0, 1.0, 0.0, 3.0])
    kv[2, lab] = bits([0.5, -0.25, 0.125, -0.0625])
    codes, scale = oracle.quantize_pair(s, kv, lab)
    assert scale[0] == 0 and codes[0].tolist() == [0, 0, 0, 0]
    assert scale[1] == np.float32(1.0) and codes[1].tolist() == [-7, 1, 0, 3]
    packed = oracle.pack_codes(codes)
    assert packed[1].tolist() == [(-7 & 0xF) | (1 << 4), 0 | (3 << 4)]
    assert packed[1].tolist() == [0x19, 0x30]


def test_quantizer_exact_ties_round_half_to_even():
    """Quotients k / scale that fall exactly half-way between two codes round to the
    even code (the reading taken for the INT4 label cache): with the label absmax at
    7 * 2^e the scale is exactly 2^e, so a key (m + 1/2) * 2^e is an exact tie.
    Half-away-from-zero would give 3 for 2.5 and -3 for -2.5; half-up would give 3 for
    2.5; truncation 2 for 2.5 but 3 for 3.5 -- each differs from the table below."""
    half_even = {0.5: 0, 1.5: 2, 2.5: 2, 3.5: 4, 4.5: 4, 5.5: 6, 6.5: 6,
                 -0.5: 0, -1.5: -2, -2.5: -2, -3.5: -4, -4.5: -4, -5.5: -6, -6.5: -6}
    s = W.small_shape(B=1, Hq=2, Hkv=1, N=2 * 3, bs=4, D=16, DV=16, r=8)
    lab = np.array([0, 2, 3, 5, 8, 11, 12, 15], dtype=np.int32)
    ties = list(half_even)
    rows, expect, scales = [], [], []
    for e in (0, -2, 3):                       # scale exactly 1, 1/4, 8
        for part in (ties[:7], ties[7:]):      # seven ties plus the +-7 channel per token
            absmax = 7.0 if part[0] > 0 else -7.0
            vals = [absmax] + part
            rows.append([v * 2.0 ** e for v in vals])
            expect.append([7 if absmax > 0 else -7] + [half_even[v] for v in part])
            scales.append(2.0 ** e)
    kv = np.zeros((len(rows), s.row), dtype=np.uint16)
    kv[:, lab] = bits(np.array(rows))
    s = s.with_(N=len(rows))
    codes, scale = oracle.quantize_pair(s, kv, lab)
    assert scale.tolist() == scales
    assert codes.tolist() == expect


# ------------------------------------------------------------ token stage --

def test_token_stage_is_exact_topk_when_codes_are_exact():
    """All channels are label channels and keys are grid-aligned per token (so the
    INT4 cache is exact): with Kb = NB, stage 2 is the exact top-Kt of max_g q_g.k."""
    s = W.small_shape(B=1, Hq=4, Hkv=1, N=500, bs=50, D=8, DV=8, r=8, Kb=10, Kt=37)
    rng = np.random.default_rng(8)
    q, _ = make_inputs(s, rng)
    m = rng.integers(-7, 8, (s.N, s.D)); m[np.arange(s.N), rng.integers(0, s.D, s.N)] = 7
    e = rng.integers(-2, 2, (s.N, 1)).astype(np.float64)
    k = (m * 2.0 ** e).astype(np.float32)
    kv = np.zeros((1, 1, s.N, s.row), dtype=np.uint16)
    kv[0, 0, :, : s.D] = bits(k)
    lab = lab_all(s)
    step = oracle.decode(s, q, kv, lab)
    dots = (f64(q[0]) @ k.astype(np.float64).T).max(axis=0)
    expect = sorted(rank_desc(dots)[: s.Kt].tolist())
    assert step.token_idx[0, : step.ntok[0]].tolist() == expect
    assert step.block_idx[0].tolist() == list(range(10))


def test_quest_only_special_case():
    """Kt = Kb*bs keeps every token of the selected blocks (block-only selection)."""
    s = W.small_shape(B=2, Hq=8, Hkv=2, N=640, bs=32, D=64, DV=64, r=8, Kb=3, Kt=96)
    rng = np.random.default_rng(9)
    q, kv = make_inputs(s, rng)
    lab = np.tile(np.arange(0, 64, 8, dtype=np.int32), (2, 1))
    step = oracle.decode(s, q, kv, lab)
    for i in range(s.pairs):
        blocks = step.block_idx[i]
        expect = sorted(int(b) * s.bs + t for b in blocks for t in range(s.bs))
        assert step.token_idx[i].tolist() == expect


# ------------------------------------------------------------- attention ---

def dense_attention_torch(s, q, kv):
    """torch's scaled_dot_product_attention in float64 over the whole cache."""
    outs, lses = [], []
    for b in range(s.B):
        for h in range(s.Hkv):
            qq = torch.from_numpy(f64(q[b, h * s.G:(h + 1) * s.G]))[None, :, None, :]
            kk = torch.from_numpy(f64(kv[b, h, :, : s.D]))
            vv = torch.from_numpy(f64(kv[b, h, :, s.v_off:s.v_off + s.DV]))
            o = torch.nn.functional.scaled_dot_product_attention(
                qq, kk[None, None].expand(1, s.G, s.N, s.D), vv[None, None].expand(1, s.G, s.N, s.DV),
                scale=s.sm_scale)
            outs.append(o[0, :, 0].numpy())
            z = (qq[0, :, 0] @ kk.T).numpy() * s.sm_scale
            lses.append(logsumexp(z, axis=1))
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("mla", [False, True])
def test_dense_when_everything_is_selected(mla):
    """Kb >= NB and Kt >= N: the two-level step equals dense attention."""
    if mla:
        s = W.small_shape(B=2, Hq=16, Hkv=1, D=72, DV=64, v_is_k_prefix=True, N=333, bs=64, r=8,
                          Kb=100, Kt=10 ** 6, n_outlier=0)
    else:
        s = W.small_shape(B=2, Hq=8, Hkv=2, N=333, bs=64, Kb=100, Kt=10 ** 6)
    rng = np.random.default_rng(12)
    q, kv = make_inputs(s, rng)
    lab = np.tile(np.arange(s.r, dtype=np.int32) * 2, (s.Hkv, 1))
    step = oracle.decode(s, q, kv, lab)
    assert np.all(step.ntok == s.N)
    ref, ref_lse = dense_attention_torch(s, q, kv)
    np.testing.assert_allclose(step.out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(step.lse, ref_lse, rtol=0, atol=1e-12)


def test_sparse_attention_matches_library_on_the_selected_rows():
    """Output over the selected tokens equals torch's dense attention over just those rows."""
    s = W.small_shape(B=1, Hq=8, Hkv=2, N=1000, bs=64, Kb=4, Kt=77)
    rng = np.random.default_rng(13)
    q, kv = make_inputs(s, rng)
    lab = np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))
    step = oracle.decode(s, q, kv, lab)
    for i in range(s.pairs):
        tok = step.token_idx[i, : step.ntok[i]]
        sub = s.with_(B=1, Hkv=1, Hq=s.G, N=tok.size)
        ref, ref_lse = dense_attention_torch(sub, q[:, i * s.G:(i + 1) * s.G], kv[:, i:i + 1, tok])
        np.testing.assert_allclose(step.out[i], ref[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(step.lse[i], ref_lse[0], rtol=0, atol=1e-12)


def test_mha_group_of_one():
    """G = 1: the max over heads is the identity; block scores equal the single head's."""
    s = W.small_shape(B=1, Hq=3, Hkv=3, N=512, bs=64, Kb=2, Kt=40)
    rng = np.random.default_rng(14)
    q, kv = make_inputs(s, rng)
    for h in range(3):
        kmax, kmin = oracle.summaries_pair(s, kv[0, h])
        _, S, s_head = oracle.select_blocks_pair(s, q[0, h:h + 1], kmax, kmin)
        np.testing.assert_array_equal(S, s_head[0])


# --------------------------------------------------------- staggered run ---

def test_zero_drift_staggered_equals_synchronous():
    """Constant q: M_t = M_{-1}, no transfers, and every step equals the synchronous step."""
    s = W.small_shape(B=2, Hq=8, Hkv=2, N=2048, bs=64, Kb=4, Kt=100, steps=5)
    rng = np.random.default_rng(15)
    q, kv = make_inputs(s, rng)
    lab = np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))
    step = oracle.decode(s, q, kv, lab)
    qs = np.repeat(q[None], 5, axis=0)
    st = oracle.staggered(s, qs, kv, lab, step)
    assert np.all(st.nT == 0) and np.all(st.nevict == 0)
    for t in range(5):
        np.testing.assert_array_equal(st.M[t], step.block_idx)
        np.testing.assert_array_equal(st.out[t], step.out)


def test_staggered_invariants_with_drift():
    """With drifting queries: T_t = M_t minus the resident set, capacity 2*Kb, step t
    uses the blocks of step t-1 (its output equals a decode forced to M_{t-1})."""
    s = W.small_shape(B=1, Hq=8, Hkv=2, N=4096, bs=64, Kb=6, Kt=128, steps=12)
    rng = np.random.default_rng(16)
    q, kv = make_inputs(s, rng)
    lab = np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))
    qs = W.drift_queries(s, q, 12)
    built = oracle.decode(s, q, kv, lab)
    st = oracle.staggered(s, qs, kv, lab, built)
    moved = 0
    for p in range(s.pairs):
        resident = set(built.block_idx[p].tolist())
        prev = built.block_idx[p].tolist()
        for t in range(12):
            stp = oracle.decode(s, qs[t], kv, lab, pairs=[p], built=_sub(built, p))
            assert st.M[t, p].tolist() == stp.block_idx[0].tolist()
            forced = oracle.decode(s, qs[t], kv, lab, pairs=[p], built=_sub(built, p), force_blocks=[prev])
            np.testing.assert_array_equal(st.out[t, p], forced.out[0])
            Tt = st.T[t, p, : st.nT[t, p]].tolist()
            assert Tt == sorted(set(st.M[t, p].tolist()) - resident)
            need = max(0, len(resident) + len(Tt) - 2 * s.Kb)
            assert st.nevict[t, p] == need
            # evicted blocks are outside M_{t-1} and M_t
            keep = set(prev) | set(st.M[t, p].tolist())
            assert len(keep) <= 2 * s.Kb
            resident = _evict_lru(resident, need, keep, p, t, st, built)
            resident |= set(Tt)
            assert len(resident) <= 2 * s.Kb
            prev = st.M[t, p].tolist()
            moved += len(Tt)
    assert moved > 0


def _drift(q0, steps, sigma, rng):
    """q_t = q_{t-1} + sigma * N(0, 1), rounded to bf16 (large sigma: many evictions)."""
    qs = np.empty((steps,) + q0.shape, dtype=np.uint16)
    qs[0] = q0
    for t in range(1, steps):
        qs[t] = W.f32_to_bf16_bits((f64(qs[t - 1]) + sigma * rng.standard_normal(q0.shape)).astype(np.float32))
    return qs


@pytest.mark.parametrize("sigma,Kb,steps", [(0.5, 4, 30), (3.0, 4, 16), (0.25, 6, 40)])
def test_staggered_lru_eviction_order(sigma, Kb, steps):
    """Schedules that evict: at every step the oracle's evicted blocks equal an LRU
    replayed here from the selection history alone -- only as many as the 2*Kb slots
    require, none of M_{t-1} or M_t, least recently selected first (the prologue
    selection counts as step -1), lower block first on equal steps."""
    s = W.small_shape(B=2, Hq=8, Hkv=2, N=2048, bs=64, Kb=Kb, Kt=64, steps=steps)
    rng = np.random.default_rng(int(sigma * 100) + Kb)
    q, kv = make_inputs(s, rng)
    lab = lab_all(s)
    qs = _drift(q, steps, sigma, rng)
    built = oracle.decode(s, qs[0], kv, lab)
    st = oracle.staggered(s, qs, kv, lab, built)
    assert st.nevict.sum() > 0
    order_matters = tie_cut = 0
    for p in range(s.pairs):
        resident = set(built.block_idx[p].tolist())
        last = {j: -1 for j in resident}
        prev = set(resident)
        for t in range(steps):
            Mt = set(st.M[t, p].tolist())
            Tt = sorted(Mt - resident)
            assert st.T[t, p, : st.nT[t, p]].tolist() == Tt
            need = max(0, len(resident) + len(Tt) - 2 * Kb)
            cands = sorted((last[j], j) for j in resident - prev - Mt)
            assert len(cands) >= need
            expect = [j for _, j in cands[:need]]
            assert st.nevict[t, p] == need
            assert st.evicted[t, p, :need].tolist() == expect, (p, t)
            if 0 < need < len(cands):
                order_matters += 1
                tie_cut += cands[need - 1][0] == cands[need][0]
            resident = (resident - set(expect)) | set(Tt)
            assert len(resident) <= 2 * Kb and Mt <= resident
            for j in Mt:
                last[j] = t
            prev = Mt
    assert order_matters > 0   # steps where a different eviction rule would pick other blocks
    if sigma >= 3.0:
        assert tie_cut > 0     # the lower-block rule decides among blocks last selected together
    # made to follow its own selections, the schedule is unchanged; made to follow
    # other (valid) selections, it applies the same rules to them
    same = oracle.staggered(s, qs, kv, lab, built, force_prologue=built.block_idx, force_M=st.M)
    for key in ("M", "T", "nT", "nevict", "evicted", "out"):
        np.testing.assert_array_equal(getattr(same, key), getattr(st, key))
    alt_M = st.M.copy()
    alt_M[1] = st.M[0]                    # step 1 repeats step 0's selection: nothing to move
    alt = oracle.staggered(s, qs, kv, lab, built, force_prologue=built.block_idx, force_M=alt_M)
    np.testing.assert_array_equal(alt.M, alt_M)
    assert np.all(alt.nT[1] == 0) and np.all(alt.nevict[1] == 0)
    np.testing.assert_array_equal(alt.out[:2], st.out[:2])   # steps 0 and 1 use M_{-1} and M_0


def _sub(built, p):
    return oracle.Step(kmax=built.kmax[p:p + 1], kmin=built.kmin[p:p + 1], codes=built.codes[p:p + 1],
                       scale=built.scale[p:p + 1])


def _evict_lru(resident, need, keep, p, t, st, built):
    """Least-recently-selected first, lower block first; selection history from st.M."""
    if need == 0:
        return resident
    def last_sel(j):
        for u in range(t, -1, -1):
            if j in st.M[u, p]:
                return u
        return -1   # the prologue selection
    cand = sorted((last_sel(j), j) for j in resident if j not in keep)
    return resident - {j for _, j in cand[:need]}


def test_generator_is_deterministic_and_bf16():
    s = W.small_shape(N=300)
    a = W.gen_kv(s); b = W.gen_kv(s)
    assert np.array_equal(a, b)
    assert np.array_equal(W.gen_kv_pair(s, 1, 1), a[1, 1])
    lab = W.label_channels(s, a[0])
    assert lab.shape == (s.Hkv, s.r) and np.all(np.diff(lab, axis=1) > 0)
    oc = W.outlier_channels(s)
    assert set(oc.tolist()) <= set(lab[0].tolist())   # x8 channels dominate mean |K|


def test_c1_regression_record():
    """The oracle still reproduces the stored 8k-context record (tests/golden/make_c1_golden.py)."""
    rec = np.load(GOLD / "c1_expected_selection.npz")
    s = W.CONFIGS["c1_8k_gqa8"]
    q = W.gen_q(s); kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    np.testing.assert_array_equal(lab, rec["label_ch"])
    st = oracle.decode(s, q, kv, lab)
    np.testing.assert_array_equal(st.block_idx, rec["block_idx"])
    np.testing.assert_array_equal(st.token_idx, rec["token_idx"])
    np.testing.assert_array_equal(st.out, rec["out"])


def test_staggered_growing_cache_equals_one_step_decodes_of_each_prefix():
    """A cache that grows between steps (lens; pages, section 1: the KV cache
    grows with every generated token). At every step t the schedule must equal a
    fresh one-step decode of the first lens[t+1] tokens alone -- summaries and
    label cache built from that prefix: its selection M_t is that decode's stage
    1, its output is that decode's attention forced to M_{t-1}; the prologue is
    stage 1 of the first lens[0] tokens. Transfers and evictions are the LRU
    replayed from the selection history, new blocks enter as the cache reaches
    them, and constant lengths give the fixed-length schedule."""
    steps = 24
    s = W.small_shape(B=1, Hq=8, Hkv=2, N=3072, bs=64, Kb=4, Kt=64, steps=steps)  # N: the allocated length
    rng = np.random.default_rng(31)
    q, kv = make_inputs(s, rng)
    lab = lab_all(s)
    qs = _drift(q, steps, 1.0, rng)
    lens = np.cumsum(np.r_[1500, rng.integers(1, 60, steps)]).astype(np.int64)
    assert lens[-1] <= s.N
    built = oracle.decode(s, qs[0], kv, lab)  # codes and scales of all N tokens
    st = oracle.staggered(s, qs, kv, lab, built, lens=lens)

    fixed = oracle.staggered(s, qs, kv, lab, built)
    const = oracle.staggered(s, qs, kv, lab, built, lens=np.full(steps + 1, s.N, dtype=np.int64))
    for f in ("M", "T", "nT", "nevict", "out", "lse"):
        np.testing.assert_array_equal(getattr(const, f), getattr(fixed, f))

    def prefix(n):
        return s.with_(N=int(n)), np.ascontiguousarray(kv[:, :, :n])

    sp, kvp = prefix(lens[0])
    prev = oracle.decode(sp, qs[0], kvp, lab).block_idx  # the prologue's M_{-1}
    history = [prev]
    for t in range(steps):
        sp, kvp = prefix(lens[t + 1])
        one = oracle.decode(sp, qs[t], kvp, lab)
        np.testing.assert_array_equal(st.M[t], one.block_idx)
        forced = oracle.decode(sp, qs[t], kvp, lab, built=one, force_blocks=prev)
        np.testing.assert_array_equal(st.out[t], forced.out)
        np.testing.assert_array_equal(st.lse[t], forced.lse)
        prev = one.block_idx
        history.append(prev)
    nb0 = (lens[0] + s.bs - 1) // s.bs
    assert (st.M >= nb0).any()  # blocks that did not exist at the prologue get selected

    # transfers and evictions: the LRU replayed from the selection history
    assert st.nevict.sum() > 0
    for p in range(s.pairs):
        resident = set(history[0][p].tolist())
        last = {j: -1 for j in resident}
        prevset = set(resident)
        for t in range(steps):
            Mt = set(history[t + 1][p].tolist())
            Tt = sorted(Mt - resident)
            assert st.T[t, p, : st.nT[t, p]].tolist() == Tt
            need = max(0, len(resident) + len(Tt) - 2 * s.Kb)
            cands = sorted((last[j], j) for j in resident - prevset - Mt)
            expect = [j for _, j in cands[:need]]
            assert st.evicted[t, p, :need].tolist() == expect, (p, t)
            resident = (resident - set(expect)) | set(Tt)
            for j in Mt:
                last[j] = t
            prevset = Mt
