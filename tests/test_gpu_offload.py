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


def run_staggered(s, q0, kv, lab, steps, helper, copy_mode=None):
    """copy_mode 3 (TLS_COPY_FULL, no reuse): the same outputs and selections,
    while every block of M_t is transferred at every step."""
    from two_level_sparse_amd.runtime import Cache, StaggeredDecoder, bf16
    qs = W.drift_queries(s, q0, steps)
    built = oracle.decode(s, q0, kv, lab)
    ref = oracle.staggered(s, qs, kv, lab, built)
    cache = Cache(s, kv, lab).build()
    host = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).pin_memory()
    sd = StaggeredDecoder(s, cache, host, bf16(q0), copy_mode=copy_mode)
    np.testing.assert_array_equal(to_np(sd.selection(-1)).reshape(s.pairs, -1), built.block_idx)
    stats = dict(moved=0, token_band=0, max_err=0.0)
    prev_blocks = built.block_idx
    for t in range(steps):
        out = sd.step(bf16(qs[t]), helper=helper)
        torch.cuda.synchronize()
        counts, blocks = sd.last_delta()
        Mt = to_np(sd.selection(t)).reshape(s.pairs, -1)
        np.testing.assert_array_equal(Mt, ref.M[t])
        if copy_mode == 3:
            np.testing.assert_array_equal(counts, np.full(s.pairs, Mt.shape[1]))
            np.testing.assert_array_equal(blocks, Mt)
        else:
            np.testing.assert_array_equal(counts, ref.nT[t])
            for p in range(s.pairs):
                assert blocks[p, : counts[p]].tolist() == ref.T[t, p, : ref.nT[t, p]].tolist()
        stats["moved"] += int(counts.sum())
        # token sets inside M_{t-1}, scored with q_t
        ti = to_np(sd.dec.token_idx).reshape(s.pairs, -1)
        for p in range(s.pairs):
            b, h = divmod(p, s.Hkv)
            _, cand, cs = oracle.select_tokens_pair(s, qs[t, b, h * s.G:(h + 1) * s.G], lab[h], built.codes[p],
                                                    built.scale[p], prev_blocks[p])
            nb, _ = band_check(ti[p], cand, cs, s.Kt)
            stats["token_band"] += nb
        o = to_np(out).reshape(s.pairs, s.G, s.DV)
        err = float(np.max(np.abs(o - ref.out[t])))
        assert err <= 2e-3, (t, err)
        stats["max_err"] = max(stats["max_err"], err)
        prev_blocks = ref.M[t]
    assert sd.total_copied() == stats["moved"]
    sd.close()
    return stats


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


def test_staggered_full_256k_offload():
    """The 256k-context offloaded workload (batch 4, 32/8 heads, Kb=128, Kt=4096),
    first 8 drift steps, every pair checked."""
    s = W.CONFIGS["c5_256k_offload"]
    print("[gpu] offload 256k: generating inputs", flush=True)
    q0 = W.gen_q(s)
    kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    st = run_staggered(s, q0, kv, lab, steps=8, helper=True)
    print(f"[gpu] staggered 256k: {st}", flush=True)


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
