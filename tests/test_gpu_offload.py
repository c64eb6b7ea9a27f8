"""GPU parity of the staggered offloaded decode (AsyncTLS pages, section 2B)
against the oracle's schedule: per step, the transferred blocks T_t, the new
selection M_t, the token sets (band rule) and the outputs (2e-3) must match."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workload as W
from gpu_common import band_check, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_level_sparse_amd as T
    T.load_library()


def run_staggered(s, q0, kv, lab, steps, helper, copy_mode=None, qs=None):
    """Runs `steps` staggered steps on the GPU, then checks them against the
    oracle's schedule (O10) made to follow the GPU's own block selections:
      - every selection M_t (and the prologue's) by the band rule on the
        oracle's block scores for q_t -- blocks of (nearly) equal score may
        legitimately differ, and the schedule after such a step is then the one
        that follows from the GPU's M_t;
      - T_t, bit-exact, against the followed schedule (so the transfers, the
        evictions behind them and the slot reuse are the oracle's);
      - the token set of step t by the band rule over M_{t-1};
      - the output within 2e-3 of the oracle's attention over the GPU's tokens.
    copy_mode 3 (TLS_COPY_FULL, no reuse): every block of M_t moves at every
    step instead. qs: the queries (default: the workload's drift, 0.1 per step)."""
    from two_level_sparse_amd.runtime import Cache, StaggeredDecoder, bf16
    if qs is None:
        qs = W.drift_queries(s, q0, steps)
    built = oracle.decode(s, q0, kv, lab)
    cache = Cache(s, kv, lab).build()
    host = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).pin_memory()
    sd = StaggeredDecoder(s, cache, host, bf16(q0), copy_mode=copy_mode)
    pro = to_np(sd.selection(-1)).reshape(s.pairs, -1).copy()
    gM, gcounts, gblocks, gtok, gout = [], [], [], [], []
    for t in range(steps):
        out = sd.step(bf16(qs[t]), helper=helper)
        torch.cuda.synchronize()
        counts, blocks = sd.last_delta()
        gM.append(to_np(sd.selection(t)).reshape(s.pairs, -1).copy())
        gcounts.append(counts.copy())
        gblocks.append(blocks.copy())
        gtok.append(to_np(sd.dec.token_idx).reshape(s.pairs, -1).copy())
        gout.append(to_np(out).reshape(s.pairs, s.G, s.DV).copy())
        if t % 16 == 15:
            print(f"[gpu] staggered: {t + 1} of {steps} steps run", flush=True)
    total = sd.total_copied()
    sd.close()
    return check_staggered(s, qs, kv, lab, built, pro, gM, gcounts, gblocks, gtok, gout, total, copy_mode)


def check_staggered(s, qs, kv, lab, built, pro, gM, gcounts, gblocks, gtok, gout, total, copy_mode=None):
    """The checks of run_staggered on one layer's recorded run (per step: M_t,
    T_t, the token set, the output; total = blocks moved)."""
    steps = len(gM)
    gM = np.stack(gM)
    own = oracle.staggered(s, qs, kv, lab, built)
    ref = oracle.staggered(s, qs, kv, lab, built, force_prologue=pro, force_M=gM)
    stats = dict(moved=0, token_band=0, block_band=0, max_err=0.0, evicted=int(ref.nevict.sum()),
                 steps_off_own_schedule=int(np.sum(np.any(gM != own.M, axis=(1, 2)))))
    for p in range(s.pairs):
        band_check(pro[p], np.arange(s.NB), built.S[p], s.Kb)
    prev_blocks = pro
    for t in range(steps):
        St = oracle.decode(s, qs[t], kv, lab, built=built).S
        counts, blocks = gcounts[t], gblocks[t]
        for p in range(s.pairs):
            nb, _ = band_check(gM[t, p], np.arange(s.NB), St[p], s.Kb)
            stats["block_band"] += nb
        if copy_mode == 3:
            np.testing.assert_array_equal(counts, np.full(s.pairs, gM.shape[2]))
            np.testing.assert_array_equal(blocks, gM[t])
        else:
            np.testing.assert_array_equal(counts, ref.nT[t])
            for p in range(s.pairs):
                assert blocks[p, : counts[p]].tolist() == ref.T[t, p, : ref.nT[t, p]].tolist(), (t, p)
        stats["moved"] += int(counts.sum())
        ti = gtok[t]
        for p in range(s.pairs):
            b, h = divmod(p, s.Hkv)
            qp = qs[t, b, h * s.G:(h + 1) * s.G]
            _, cand, cs = oracle.select_tokens_pair(s, qp, lab[h], built.codes[p], built.scale[p], prev_blocks[p])
            nb, _ = band_check(ti[p], cand, cs, s.Kt)
            stats["token_band"] += nb
            o_ref, _ = oracle.attend_pair(s, qp, kv[b, h], ti[p][ti[p] >= 0])
            err = float(np.max(np.abs(gout[t][p] - o_ref)))
            assert err <= 2e-3, (t, p, err)
            stats["max_err"] = max(stats["max_err"], err)
        prev_blocks = gM[t]
    assert total == stats["moved"]
    return stats


@pytest.mark.parametrize("mode", [2, 1])
def test_layered_staggered_decode(mode):
    """Three layers, each its own offloaded cache and query sequence, stepped
    as one model (LayeredDecoder: shared stage and copy streams, layer l+1's
    selection after layer l's attention): every layer against the oracle's
    schedule for its own inputs, as in run_staggered. Device planning is also
    captured as one graph of all layers' steps and replayed, with the same
    outputs."""
    from two_level_sparse_amd.runtime import Cache, LayeredDecoder, bf16
    L, steps = 3, 12
    shapes = [W.small_shape(B=2, Hq=8, Hkv=2, N=8192, bs=64, Kb=8, Kt=200, n_outlier=4, seed=60 + l) for l in range(L)]
    q0s = [W.gen_q(sl) for sl in shapes]
    kvs = [W.gen_kv(sl) for sl in shapes]
    labs = [W.label_channels(sl, kv[0]) for sl, kv in zip(shapes, kvs)]
    qss = [W.drift_queries(sl, q0, steps) for sl, q0 in zip(shapes, q0s)]
    s = shapes[0]
    caches = [Cache(sl, kv, lab).build() for sl, kv, lab in zip(shapes, kvs, labs)]
    hosts = [torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).pin_memory() for kv in kvs]
    ld = LayeredDecoder(s, caches, hosts, [bf16(q0) for q0 in q0s], copy_mode=mode)
    pros = [to_np(d.selection(-1)).reshape(s.pairs, -1).copy() for d in ld.layers]
    rec = [dict(M=[], counts=[], blocks=[], tok=[], out=[]) for _ in range(L)]
    for t in range(steps):
        outs = ld.step([bf16(qss[l][t]) for l in range(L)])
        torch.cuda.synchronize()
        for l, d in enumerate(ld.layers):
            counts, blocks = d.last_delta()
            rec[l]["M"].append(to_np(d.selection(t)).reshape(s.pairs, -1).copy())
            rec[l]["counts"].append(counts.copy())
            rec[l]["blocks"].append(blocks.copy())
            rec[l]["tok"].append(to_np(d.dec.token_idx).reshape(s.pairs, -1).copy())
            rec[l]["out"].append(to_np(outs[l]).reshape(s.pairs, s.G, s.DV).copy())
    totals = [d.total_copied() for d in ld.layers]
    ld.close()
    for l in range(L):
        built = oracle.decode(shapes[l], q0s[l], kvs[l], labs[l])
        r = rec[l]
        check_staggered(shapes[l], qss[l], kvs[l], labs[l], built, pros[l], r["M"], r["counts"], r["blocks"],
                        r["tok"], r["out"], totals[l], mode)
    if mode == 2:  # the same steps as one graph of every layer
        ld = LayeredDecoder(s, caches, hosts, [bf16(q0) for q0 in q0s], copy_mode=mode)
        qd = [[bf16(qss[l][t]) for l in range(L)] for t in range(steps)]
        outs = [torch.empty((s.B, s.Hq, s.DV), dtype=torch.float32, device="cuda") for _ in range(L)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            main = torch.cuda.current_stream()
            for t in range(steps):
                res = ld.step(qd[t])
                if t == steps - 1:
                    for l in range(L):
                        outs[l].copy_(res[l])
            main.wait_stream(ld.stage)
            main.wait_stream(ld.side)
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            np.testing.assert_array_equal(to_np(outs[l]).reshape(s.pairs, s.G, s.DV), rec[l]["out"][-1])
        ld.close()


@pytest.mark.parametrize("mode", [2, 0, 1])
def test_staggered_growing_cache(mode):
    """A cache that grows between steps (tls_offload_append: 1-63 rows before
    each step, across block boundaries and into new blocks) against the
    oracle's schedule over the same lengths, made to follow the GPU's own
    selections: every M_t (band rule on the block scores of the prefix), T_t
    bit-exact, token sets by the band rule, outputs within 2e-3 of attention
    over the GPU's tokens; afterwards the index (summaries, codes, scales) is
    bit-exact against the oracle's build of the grown cache and the host cache
    holds the appended rows. Device planning (2) and both host-planned modes."""
    import two_level_sparse_amd as T
    from gpu_common import bf16_bits, unpack_summaries
    from two_level_sparse_amd.runtime import GrowingCache, StaggeredDecoder, bf16
    steps, cap, N0 = 24, 6144, 3000
    s_cap = W.small_shape(B=2, Hq=8, Hkv=2, N=cap, bs=64, Kb=8, Kt=200, n_outlier=4, seed=41)
    q0 = W.gen_q(s_cap)
    kv = W.gen_kv(s_cap)
    lab = W.label_channels(s_cap, kv[0])
    rng = np.random.default_rng(41)
    adds = rng.integers(1, 64, steps)
    adds[5] = 64  # a whole block at once
    lens = np.cumsum(np.r_[N0, adds]).astype(np.int64)
    assert lens[-1] <= cap
    qs = W.drift_queries(s_cap, q0, steps)
    s0 = s_cap.with_(N=N0)
    gc = GrowingCache(s0, kv[:, :, :N0], lab, cap).build()
    host = torch.zeros((s_cap.B, s_cap.Hkv, cap, s_cap.row), dtype=torch.bfloat16).pin_memory()
    host[:, :, :N0] = torch.from_numpy(kv[:, :, :N0].view(np.int16)).view(torch.bfloat16)
    sd = StaggeredDecoder(s0, gc, host, bf16(q0), copy_mode=mode)
    assert sd.copy_mode == mode
    pro = to_np(sd.selection(-1)).reshape(s_cap.pairs, -1).copy()
    gM, gcounts, gblocks, gtok, gout = [], [], [], [], []
    for t in range(steps):
        sd.append(bf16(np.ascontiguousarray(kv[:, :, lens[t]:lens[t + 1]])))
        out = sd.step(bf16(qs[t]))
        torch.cuda.synchronize()
        counts, blocks = sd.last_delta()
        gM.append(to_np(sd.selection(t)).reshape(s_cap.pairs, -1).copy())
        gcounts.append(counts.copy())
        gblocks.append(blocks.copy())
        gtok.append(to_np(sd.dec.token_idx).reshape(s_cap.pairs, -1).copy())
        gout.append(to_np(out).reshape(s_cap.pairs, s_cap.G, s_cap.DV).copy())
    assert sd.n == lens[-1]
    sd.close()
    gM = np.stack(gM)
    built = oracle.decode(s_cap, q0, kv, lab)  # codes and scales of every token
    ref = oracle.staggered(s_cap, qs, kv, lab, built, force_prologue=pro, force_M=gM, lens=lens)

    def prefix(n):
        return s_cap.with_(N=int(n)), np.ascontiguousarray(kv[:, :, :n])

    sp, kvp = prefix(lens[0])
    S0 = oracle.decode(sp, q0, kvp, lab).S
    for p in range(s_cap.pairs):
        band_check(pro[p], np.arange(sp.NB), S0[p], s_cap.Kb)
    prev_blocks = pro
    new_blocks = 0
    for t in range(steps):
        sp, kvp = prefix(lens[t + 1])
        one = oracle.decode(sp, qs[t], kvp, lab)
        for p in range(s_cap.pairs):
            band_check(gM[t, p], np.arange(sp.NB), one.S[p], s_cap.Kb)
            assert gblocks[t][p, : gcounts[t][p]].tolist() == ref.T[t, p, : ref.nT[t, p]].tolist(), (t, p)
            b, h = divmod(p, s_cap.Hkv)
            qp = qs[t, b, h * s_cap.G:(h + 1) * s_cap.G]
            ti = gtok[t][p]
            _, cand, cs = oracle.select_tokens_pair(sp, qp, lab[h], one.codes[p], one.scale[p], prev_blocks[p])
            band_check(ti, cand, cs, s_cap.Kt)
            assert ti.max() < lens[t + 1]
            o_ref, _ = oracle.attend_pair(sp, qp, kv[b, h], ti[ti >= 0])
            assert float(np.max(np.abs(gout[t][p] - o_ref))) <= 2e-3, (t, p)
        new_blocks += int(np.sum(gM[t] >= (lens[0] + s_cap.bs - 1) // s_cap.bs))
        prev_blocks = gM[t]
    assert new_blocks > 0  # blocks that did not exist at the start were selected and moved
    # the index of the grown cache and the host rows
    n = int(lens[-1])
    sn, kvn = prefix(n)
    fin = oracle.decode(sn, q0, kvn, lab)
    summ = unpack_summaries(gc.summ, s_cap, sn.NB)
    for p in range(s_cap.pairs):
        np.testing.assert_array_equal(W.bf16_bits_to_f64(summ[p, :, 0]), fin.kmax[p])
        np.testing.assert_array_equal(W.bf16_bits_to_f64(summ[p, :, 1]), fin.kmin[p])
    codes = to_np(gc.codes).reshape(s_cap.pairs, cap, -1)[:, :n]
    scale = to_np(gc.scale).reshape(s_cap.pairs, cap)[:, :n]
    for p in range(s_cap.pairs):
        np.testing.assert_array_equal(codes[p], oracle.pack_codes(fin.codes[p]))
        np.testing.assert_array_equal(scale[p].view(np.uint32), fin.scale[p].view(np.uint32))
    np.testing.assert_array_equal(host.view(torch.int16).numpy().view(np.uint16)[:, :, :n], kv[:, :, :n])


@pytest.mark.parametrize("helper,mode", [(False, 1), (True, 1), (False, 0), (True, 0), (False, 2), (True, 2), (False, 3)])
def test_staggered_small(helper, mode):
    s = W.small_shape(B=2, Hq=8, Hkv=2, N=8192, bs=64, Kb=8, Kt=200, n_outlier=4, seed=21)
    rng = np.random.default_rng(21)
    q0 = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
    k = rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32)
    k[..., :4] *= 8
    kv = W.f32_to_bf16_bits(k)
    lab = np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))
    st = run_staggered(s, q0, kv, lab, steps=16, helper=helper, copy_mode=mode)
    print(f"[gpu] staggered small helper={helper} copy_mode={mode}: {st}", flush=True)
    assert st["moved"] > 0


@pytest.mark.parametrize("helper,mode", [(False, 1), (True, 0), (False, 2)])
def test_staggered_many_evictions(helper, mode):
    """Large query drift (q_t = q_{t-1} + N(0, 1)): most of M_t changes at every
    step, so every step evicts several blocks and the least-recently-selected
    order (lower block on ties) decides which; each copy mode against the
    oracle's schedule."""
    s = W.small_shape(B=2, Hq=8, Hkv=2, N=8192, bs=64, Kb=8, Kt=200, n_outlier=4, seed=22)
    rng = np.random.default_rng(22)
    q0 = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
    kv = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32))
    lab = np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))
    steps = 20
    qs = np.empty((steps,) + q0.shape, dtype=np.uint16)
    qs[0] = q0
    for t in range(1, steps):
        qs[t] = W.f32_to_bf16_bits((W.bf16_bits_to_f64(qs[t - 1]) + rng.standard_normal(q0.shape))
                                   .astype(np.float32))
    st = run_staggered(s, q0, kv, lab, steps=steps, helper=helper, copy_mode=mode, qs=qs)
    print(f"[gpu] staggered many evictions helper={helper} copy_mode={mode}: {st}", flush=True)
    assert st["evicted"] >= 4 * steps


def test_staggered_full_256k_offload():
    """The 256k-context offloaded workload (batch 4, 32/8 heads, Kb=128, Kt=4096)
    over all 64 drift steps the benchmark runs, every pair checked."""
    s = W.CONFIGS["c5_256k_offload"]
    print("[gpu] offload 256k: generating inputs", flush=True)
    q0 = W.gen_q(s)
    kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    st = run_staggered(s, q0, kv, lab, steps=s.steps, helper=True)
    print(f"[gpu] staggered 256k: {st}", flush=True)
    assert st["evicted"] > 0


def small_context():
    from two_level_sparse_amd.runtime import Cache, StaggeredDecoder, bf16
    s = W.small_shape(B=1, Hq=4, Hkv=2, N=4096, bs=64, Kb=4, Kt=64, n_outlier=2, seed=5)
    rng = np.random.default_rng(5)
    q0 = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
    kv = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32))
    lab = np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))
    cache = Cache(s, kv, lab).build()
    host = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).pin_memory()
    return s, q0, StaggeredDecoder(s, cache, host, bf16(q0))


def test_device_planning_is_the_default_and_fixed_after_step_0():
    import two_level_sparse_amd as T
    from two_level_sparse_amd.runtime import bf16
    s, q0, sd = small_context()
    assert sd.copy_mode == T.TLS_COPY_DEVICE
    T.tls_offload_set_copy_mode(sd.ctx, T.TLS_COPY_GATHER)  # before step 0: allowed
    T.tls_offload_set_copy_mode(sd.ctx, T.TLS_COPY_DEVICE)
    sd.step(bf16(q0))
    torch.cuda.synchronize()
    with pytest.raises(T.TlsError) as ei:
        T.tls_offload_set_copy_mode(sd.ctx, T.TLS_COPY_GATHER)
    assert ei.value.code == T.TLS_ERR_STATE
    sd.close()


def test_device_planning_rejects_an_invalid_selection():
    """A block number outside [0, NB) in M_t: the planning kernel changes
    nothing and the next host query reports it."""
    import two_level_sparse_amd as T
    s, q0, sd = small_context()
    bad = sd.selection(-1).clone()
    bad.view(-1)[1] = s.NB + 3
    map_before = sd.maps[1].clone()
    ev = torch.cuda.Event()
    ev.record()  # creates the HIP event
    T.tls_prefetch_delta(sd.ctx, 0, bad, sd.side, ev)
    torch.cuda.synchronize()
    with pytest.raises(T.TlsError) as ei:
        sd.total_copied()
    assert ei.value.code == T.TLS_ERR_STATE
    # the map of step 1 is the map of step 0 for every pair
    assert torch.equal(sd.maps[1], sd.maps[0])
    assert torch.equal(map_before, sd.maps[0])
    sd.close()


@pytest.mark.parametrize("mode", [0, 1])
def test_host_planning_rejects_an_invalid_selection_before_changing_state(mode):
    """Host-planned modes: M_t valid for pair 0 but not for pair 1 -- the call
    fails and changes nothing, so retrying the step with a valid M_t gives what
    a fresh context gives for it (transfers, slot maps, blocks moved)."""
    import two_level_sparse_amd as T
    s, q0, sd_a = small_context()
    _, _, sd_b = small_context()
    pro = to_np(sd_a.selection(-1)).reshape(s.pairs, -1)
    good = pro.copy()
    for p in range(s.pairs):  # one block of each pair's set replaced by one outside it
        outside = np.setdiff1d(np.arange(s.NB), pro[p])
        good[p, -1] = outside[-1]
        good[p] = np.sort(good[p])
    bad = good.copy()
    bad[1, 0] = -5
    for sd in (sd_a, sd_b):
        T.tls_offload_set_copy_mode(sd.ctx, mode)
    ev = torch.cuda.Event()
    ev.record()  # creates the HIP event
    dgood = torch.from_numpy(good.astype(np.int32)).cuda()
    dbad = torch.from_numpy(bad.astype(np.int32)).cuda()
    torch.cuda.synchronize()
    with pytest.raises(T.TlsError) as ei:
        T.tls_prefetch_delta(sd_a.ctx, 0, dbad, sd_a.side, ev)
    assert ei.value.code == T.TLS_ERR_STATE
    assert sd_a.total_copied() == 0
    n_a = T.tls_prefetch_delta(sd_a.ctx, 0, dgood, sd_a.side, ev)
    n_b = T.tls_prefetch_delta(sd_b.ctx, 0, dgood, sd_b.side, ev)
    torch.cuda.synchronize()
    assert n_a == n_b == s.pairs
    ca, ba = sd_a.last_delta()
    cb, bb = sd_b.last_delta()
    np.testing.assert_array_equal(ca, cb)
    np.testing.assert_array_equal(ba, bb)
    assert torch.equal(sd_a.maps[1], sd_b.maps[1])
    sd_a.close()
    sd_b.close()


def test_staggered_graph_replay_matches_the_oracle():
    """The same staggered steps captured into one HIP graph (device planning)
    and replayed: every step's output, the last selection and delta, and the
    total transfer match the oracle's schedule."""
    from two_level_sparse_amd.runtime import Cache, StaggeredDecoder, bf16
    s = W.small_shape(B=2, Hq=8, Hkv=2, N=8192, bs=64, Kb=8, Kt=200, n_outlier=4, seed=23)
    rng = np.random.default_rng(23)
    q0 = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
    k = rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32)
    k[..., :4] *= 8
    kv = W.f32_to_bf16_bits(k)
    lab = np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))
    steps = 12
    qs = W.drift_queries(s, q0, steps)
    ref = oracle.staggered(s, qs, kv, lab, oracle.decode(s, q0, kv, lab))
    cache = Cache(s, kv, lab).build()
    host = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).pin_memory()
    sd = StaggeredDecoder(s, cache, host, bf16(q0))
    qd = [bf16(qs[t]) for t in range(steps)]
    outs = [torch.empty((s.B, s.Hq, s.DV), dtype=torch.float32, device="cuda") for _ in range(steps)]
    print("[gpu] staggered graph: capture", flush=True)
    g = sd.capture(qd, outs)
    torch.cuda.synchronize()
    print("[gpu] staggered graph: replay", flush=True)
    g.replay()
    torch.cuda.synchronize()
    errs = []
    for t in range(steps):
        o = to_np(outs[t]).reshape(s.pairs, s.G, s.DV)
        errs.append(float(np.max(np.abs(o - ref.out[t]))))
    print(f"[gpu] staggered graph: max err per step {max(errs):.2e}", flush=True)
    assert max(errs) <= 2e-3, errs
    np.testing.assert_array_equal(to_np(sd.selection(steps - 1)).reshape(s.pairs, -1), ref.M[steps - 1])
    counts, blocks = sd.last_delta()
    np.testing.assert_array_equal(counts, ref.nT[steps - 1])
    for p in range(s.pairs):
        assert blocks[p, : counts[p]].tolist() == ref.T[steps - 1, p, : ref.nT[steps - 1, p]].tolist()
    assert sd.total_copied() == int(ref.nT.sum())
    sd.close()


@pytest.mark.parametrize("mode", [2, 0])
def test_in_order_steps_match_the_synchronous_decode(mode):
    """The baseline without staggering: step t selects M_t, moves the same delta
    T_t as the staggered schedule, and attends over tokens of M_t -- the
    synchronous decode of q_t (oracle) at every step."""
    from two_level_sparse_amd.runtime import Cache, StaggeredDecoder, bf16
    s = W.small_shape(B=2, Hq=8, Hkv=2, N=8192, bs=64, Kb=8, Kt=200, n_outlier=4, seed=24)
    rng = np.random.default_rng(24)
    q0 = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
    k = rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32)
    k[..., :4] *= 8
    kv = W.f32_to_bf16_bits(k)
    lab = np.tile(np.arange(s.r, dtype=np.int32), (s.Hkv, 1))
    steps = 10
    qs = W.drift_queries(s, q0, steps)
    built = oracle.decode(s, q0, kv, lab)
    ref = oracle.staggered(s, qs, kv, lab, built)
    cache = Cache(s, kv, lab).build()
    host = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).pin_memory()
    sd = StaggeredDecoder(s, cache, host, bf16(q0), copy_mode=mode, stagger=False)
    worst = 0.0
    for t in range(steps):
        out = sd.step(bf16(qs[t]))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(sd.selection(t)).reshape(s.pairs, -1), ref.M[t])
        counts, blocks = sd.last_delta()
        np.testing.assert_array_equal(counts, ref.nT[t])
        for p in range(s.pairs):
            assert blocks[p, : counts[p]].tolist() == ref.T[t, p, : ref.nT[t, p]].tolist()
        ti = to_np(sd.dec.token_idx).reshape(s.pairs, -1)
        o = to_np(out).reshape(s.pairs, s.G, s.DV)
        for p in range(s.pairs):
            b, h = divmod(p, s.Hkv)
            qp = qs[t, b, h * s.G:(h + 1) * s.G]
            _, cand, cs = oracle.select_tokens_pair(s, qp, lab[h], built.codes[p], built.scale[p], ref.M[t][p])
            band_check(ti[p], cand, cs, s.Kt)
            ref_o, _ = oracle.attend_pair(s, qp, kv[b, h], ti[p][ti[p] >= 0])
            worst = max(worst, float(np.max(np.abs(o[p] - ref_o))))
    print(f"[gpu] in-order steps mode {mode}: max err {worst:.2e}", flush=True)
    assert worst <= 2e-3
    sd.close()
