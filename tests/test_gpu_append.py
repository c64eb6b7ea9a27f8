"""GPU parity of decode-time appends (tls_append_kv) against the oracle.

A cache allocated for more tokens than it holds grows by appends of 1 to 130
rows per call, across block boundaries and from a ragged last block. After
every append the summaries of all blocks, the codes and the scales must equal
the oracle's for the grown length bit for bit (the pages' block summaries and
INT4 label cache of the longer sequence). Then one decode step through the
capacity-strided buffers is checked like any other: block and token sets
within the score band, outputs within 2e-3 of the oracle's attention over the
same token sets."""
import numpy as np
import pytest
import torch

import oracle
import workload as W
from gpu_common import band_check, bf16_bits, to_np, unpack_summaries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_level_sparse_amd as T
    T.load_library()


CASES = {
    # name: (final shape, initial length, capacity, rows per append)
    "gqa": (W.small_shape(B=2, Hq=8, Hkv=2, N=1233, bs=64, Kb=6, Kt=160, seed=31), 1000, 1300,
            [1, 1, 37, 64, 130]),
    "gqa_bs16": (W.small_shape(B=1, Hq=4, Hkv=1, N=600, bs=16, Kb=12, Kt=64, seed=32), 512, 640, [1, 16, 17, 54]),
    "mla": (W.small_shape(B=1, Hq=16, Hkv=1, D=576, DV=512, v_is_k_prefix=True, N=333, bs=64, r=32, Kb=3, Kt=100,
                          n_outlier=0, seed=33), 200, 400, [1, 63, 69]),
}


def check_indices(s, gc, kv, lab, n):
    """summaries, codes and scales of the first n tokens against the oracle's build of length n"""
    sn = s.with_(N=n)
    summ = unpack_summaries(gc.summ, s, sn.NB)
    codes = to_np(gc.codes).reshape(s.pairs, -1, s.r // 2)[:, :n]
    scale = to_np(gc.scale).reshape(s.pairs, -1)[:, :n]
    rows = bf16_bits(gc.kv).reshape(s.pairs, -1, s.row)[:, :n]
    for p in range(s.pairs):
        b, h = divmod(p, s.Hkv)
        kvp = kv[b, h, :n]
        np.testing.assert_array_equal(rows[p], kvp)
        kmax, kmin = oracle.summaries_pair(sn, kvp)
        np.testing.assert_array_equal(W.bf16_bits_to_f64(summ[p, :, 0]), kmax)
        np.testing.assert_array_equal(W.bf16_bits_to_f64(summ[p, :, 1]), kmin)
        c, sc = oracle.quantize_pair(sn, kvp, lab[h])
        np.testing.assert_array_equal(codes[p], oracle.pack_codes(c))
        np.testing.assert_array_equal(scale[p].view(np.uint32), sc.view(np.uint32))


@pytest.mark.parametrize("name", list(CASES))
def test_append_then_decode(name):
    from two_level_sparse_amd.runtime import Decoder, GrowingCache, bf16
    s, n0, cap, appends = CASES[name]
    assert n0 + sum(appends) == s.N
    print(f"[gpu] append {name}: N {n0} -> {s.N}, capacity {cap}", flush=True)
    q = W.gen_q(s)
    kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    gc = GrowingCache(s.with_(N=n0), kv[:, :, :n0], lab, cap).build()
    torch.cuda.synchronize()
    check_indices(s, gc, kv, lab, n0)
    n = n0
    for k in appends:
        gc.append(bf16(kv[:, :, n:n + k]))
        n += k
        torch.cuda.synchronize()
        assert gc.n == n
        check_indices(s, gc, kv, lab, n)

    # one decode step through the capacity-strided cache
    dec = Decoder(s.with_(N=cap))
    assert dec.kb == min(s.Kb, s.NB) and dec.kt == min(s.Kt, dec.kb * s.bs)
    dec.select_blocks(bf16(q), gc, keep_scores=False, shape=gc.shape)
    dec.select_tokens(bf16(q), gc, shape=gc.shape)
    dec.decode(bf16(q), gc.kv, shape=gc.shape)
    torch.cuda.synchronize()
    ref = oracle.decode(s, q, kv, lab)
    gb = to_np(dec.block_idx).reshape(s.pairs, -1)
    gt = to_np(dec.token_idx).reshape(s.pairs, -1)
    out = to_np(dec.out).reshape(s.pairs, s.G, s.DV)
    worst = 0.0
    for p in range(s.pairs):
        b, h = divmod(p, s.Hkv)
        band_check(gb[p], np.arange(s.NB), ref.S[p], dec.kb)
        qp = q[b, h * s.G:(h + 1) * s.G]
        _, cand, cs = oracle.select_tokens_pair(s, qp, lab[h], ref.codes[p], ref.scale[p], gb[p])
        band_check(gt[p], cand, cs, s.Kt)
        o, _ = oracle.attend_pair(s, qp, kv[b, h], gt[p][gt[p] >= 0])
        worst = max(worst, float(np.max(np.abs(out[p] - o))))
    print(f"[gpu] append {name}: decode max err {worst:.2e}", flush=True)
    assert worst <= 2e-3
