"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every stage is compared on identical inputs (the oracle's block sets feed the
GPU token stage, the oracle's token sets feed the GPU attention), then the
whole GPU chain is checked against oracle attention on the GPU's own sets.
Summaries, INT4 codes and scales must be bit-exact; index sets follow the
1e-5 relative band rule; outputs must be within 2e-3 max-abs.
"""
import sys

import zlib

import numpy as np
import pytest
import torch

import oracle
import workload as W
from gpu_common import GpuRun, band_check, check_all, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_level_sparse_amd as T
    T.load_library()   # fails loudly when the HIP library is missing


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(s, int_range=None, seed=0):
    rng = np.random.default_rng(seed)
    if int_range is None:
        q = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
        k = rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32)
        oc = rng.permutation(s.D)[: s.n_outlier]
        k[..., oc] *= 8
        kv = W.f32_to_bf16_bits(k)
    else:
        q = W.f32_to_bf16_bits(rng.integers(-int_range, int_range + 1, (s.B, s.Hq, s.D)).astype(np.float32))
        kv = W.f32_to_bf16_bits(rng.integers(-int_range, int_range + 1, (s.B, s.Hkv, s.N, s.row)).astype(np.float32))
    lab = np.stack([np.sort(rng.choice(s.D, s.r, replace=False)) for _ in range(s.Hkv)]).astype(np.int32)
    return q, kv, lab


SMALL = {
    "gqa8_ragged": W.small_shape(B=2, Hq=16, Hkv=2, N=1000, bs=64, Kb=5, Kt=200),
    "gqa4": W.small_shape(B=3, Hq=16, Hkv=4, N=4096, bs=64, Kb=8, Kt=300),
    "mha": W.small_shape(B=2, Hq=3, Hkv=3, N=2500, bs=64, Kb=6, Kt=128),
    "g12": W.small_shape(B=1, Hq=24, Hkv=2, N=3000, bs=64, Kb=7, Kt=333),
    "g32_d64_bs16": W.small_shape(B=2, Hq=64, Hkv=2, D=64, DV=64, N=777, bs=16, r=8, Kb=10, Kt=50),
    "d256_bs32": W.small_shape(B=2, Hq=8, Hkv=1, D=256, DV=256, N=1500, bs=32, r=32, Kb=9, Kt=100),
    "mla_small": W.small_shape(B=2, Hq=128, Hkv=1, D=576, DV=512, v_is_k_prefix=True, N=2048, bs=64, r=32,
                               Kb=8, Kt=256, n_outlier=0),
    "select_all": W.small_shape(B=1, Hq=8, Hkv=2, N=900, bs=64, Kb=1000, Kt=100000),
    "k_one": W.small_shape(B=2, Hq=8, Hkv=2, N=1024, bs=64, Kb=1, Kt=1),
    "many_splits": W.small_shape(B=1, Hq=8, Hkv=1, N=65536, bs=64, Kb=200, Kt=9000),
    "bs1": W.small_shape(B=1, Hq=4, Hkv=1, N=300, bs=1, D=64, DV=64, r=8, Kb=40, Kt=17),
    # token selection over more than 16384 candidates (passes over chunks):
    # two passes; four passes (70016 -> 40000 -> 24000 -> 16000 -> 8000)
    "ds_two_pass": W.small_shape(B=1, Hq=8, Hkv=2, N=40000, bs=64, Kb=1000, Kt=3000),
    "ds_four_pass": W.small_shape(B=1, Hq=4, Hkv=1, N=70000, bs=64, Kb=2000, Kt=8000),
    # token selection at its limits: exactly 16384 candidates (16 per thread
    # of one 1024-thread selection); label-channel counts whose codes load
    # byte by byte (r = 12 with 8 heads, r = 20 with 128); 1100 kept blocks of 8
    "cand_16384": W.small_shape(B=1, Hq=8, Hkv=2, N=20000, bs=64, Kb=256, Kt=5000),
    "r12": W.small_shape(B=2, Hq=16, Hkv=2, N=3000, bs=64, r=12, Kb=10, Kt=300),
    "g128_r20": W.small_shape(B=1, Hq=128, Hkv=1, D=576, DV=512, v_is_k_prefix=True, N=3000, bs=64, r=20,
                              Kb=12, Kt=400, n_outlier=0),
    "bs8_1100_blocks": W.small_shape(B=1, Hq=8, Hkv=1, N=10000, bs=8, Kb=1100, Kt=2000),
    # folded token scores (two candidate tiles per MFMA) with 8 label channels
    # and 4 heads, a ragged last block
    "r8_g4_fold": W.small_shape(B=2, Hq=8, Hkv=2, N=3000, bs=64, r=8, Kb=10, Kt=300),
    # tls_select's block top-k inside the token scorer: up to 4096 blocks (16
    # per thread at most; 9 at 2188), and the separate block top-k above (4375)
    "nb_2188": W.small_shape(B=1, Hq=8, Hkv=1, N=140000, bs=64, Kb=40, Kt=1000),
    "nb_4375_bs16": W.small_shape(B=1, Hq=8, Hkv=1, N=70000, bs=16, Kb=100, Kt=800),
    # degenerate lengths: one cached token; fewer tokens than one block
    "n_one": W.small_shape(B=2, Hq=8, Hkv=2, N=1, bs=64, Kb=4, Kt=16),
    "n_below_block": W.small_shape(B=1, Hq=8, Hkv=1, N=37, bs=64, Kb=3, Kt=20),
    # head groups above 48 take the LDS-staged block scorer: 4 tiles of 16
    # blocks per workgroup, ragged tile counts and head tiles past G
    "g64_lds": W.small_shape(B=1, Hq=128, Hkv=2, N=3000, bs=32, Kb=12, Kt=200),
    "g80_d256": W.small_shape(B=1, Hq=80, Hkv=1, D=256, DV=256, N=1500, bs=16, Kb=20, Kt=150),
    "g100_d64": W.small_shape(B=2, Hq=100, Hkv=1, D=64, DV=64, N=5000, bs=64, r=8, Kb=9, Kt=300),
    # latent attention on MFMA: a half-empty second head group, 16 splits of one tile
    "mla_g48": W.small_shape(B=1, Hq=48, Hkv=1, D=576, DV=512, v_is_k_prefix=True, N=3000, bs=32, r=32,
                             Kb=20, Kt=500, n_outlier=0),
    # tls_select scoring the blocks inside the token stage at its limit (384
    # blocks per pair), and one token past it (385 blocks, the last holding
    # one token: the separate block scorer)
    "nb_384_inside": W.small_shape(B=1, Hq=16, Hkv=2, N=384 * 64, bs=64, Kb=40, Kt=1000),
    "nb_385_ragged": W.small_shape(B=1, Hq=16, Hkv=2, N=384 * 64 + 1, bs=64, Kb=40, Kt=1000),
    # pair counts that are a multiple of 8: the token scorers place all of a
    # pair's workgroups on one XCD (their pair/unit mapping is permuted)
    "pairs8_gqa": W.small_shape(B=4, Hq=16, Hkv=2, N=3000, bs=64, Kb=10, Kt=300),
    "pairs8_mla": W.small_shape(B=8, Hq=128, Hkv=1, D=576, DV=512, v_is_k_prefix=True, N=1000, bs=64, r=32,
                                Kb=6, Kt=200, n_outlier=0),
    # few heads on the 576-wide rows: the vector attention kernel
    "mla_g8": W.small_shape(B=2, Hq=8, Hkv=1, D=576, DV=512, v_is_k_prefix=True, N=1500, bs=64, r=32,
                            Kb=6, Kt=200, n_outlier=0),
    # the workgroup's shared gather of q on the label channels at the ends of
    # its range: the fewest channels (r = 2, 30 of 32 slots padding) and all
    # 32 slots on three head tiles, the last one ragged (G = 40)
    "r2_g16": W.small_shape(B=1, Hq=32, Hkv=2, N=1500, bs=64, r=2, Kb=6, Kt=100),
    "r32_g40": W.small_shape(B=1, Hq=40, Hkv=1, N=2000, bs=64, r=32, Kb=8, Kt=200),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_shapes(name):
    s = SMALL[name]
    log(f"[gpu] small shape {name}: {s}")
    q, kv, lab = inputs(s, seed=zlib.crc32(name.encode()) % 1000)  # the same seed in every process
    st = check_all(s, q, kv, lab)
    log(f"[gpu] {name}: {st}")


def test_latent_attention_over_every_token():
    """The latent-attention kernel at its split limit: 32 heads on one 576-dim
    kv row attend over all 49152 cached tokens (128 splits of 384 tokens, the
    dense baseline's shape), against the oracle's attention over the same
    tokens."""
    from two_level_sparse_amd.runtime import Decoder, bf16
    s = W.small_shape(B=1, Hq=32, Hkv=1, D=576, DV=512, v_is_k_prefix=True, N=49152, bs=64, r=32, Kb=768,
                      Kt=49152, n_outlier=0, seed=41)
    log(f"[gpu] latent attention over every token: {s}")
    rng = np.random.default_rng(41)
    q = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
    kv = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32))
    dec = Decoder(s)
    idx = torch.arange(s.N, dtype=torch.int32, device="cuda").view(1, 1, -1).contiguous()
    dec.decode(bf16(q), bf16(kv), token_idx=idx)
    torch.cuda.synchronize()
    out = to_np(dec.out).reshape(s.G, s.DV)
    lse = to_np(dec.lse).reshape(s.G)
    o_ref, l_ref = oracle.attend_pair(s, q[0], kv[0, 0], np.arange(s.N))
    err = float(np.max(np.abs(out - o_ref)))
    log(f"[gpu] latent attention over every token: max err {err:.2e}")
    assert err <= 2e-3
    assert np.max(np.abs(lse - l_ref)) <= 2e-3


def test_gqa_attention_over_every_token():
    """The 128-channel attention kernel at its split limits: 8 heads on one kv
    head attend over all 131072 cached tokens (64 splits of 2048 tokens, the
    dense baseline's per-pair shape at 128k), against the oracle's attention
    over the same tokens."""
    from two_level_sparse_amd.runtime import Decoder, bf16
    s = W.small_shape(B=1, Hq=8, Hkv=1, D=128, DV=128, N=131072, bs=64, r=16, Kb=2048, Kt=131072, seed=43)
    log(f"[gpu] 128-channel attention over every token: {s}")
    rng = np.random.default_rng(43)
    q = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hq, s.D)).astype(np.float32))
    kv = W.f32_to_bf16_bits(rng.standard_normal((s.B, s.Hkv, s.N, s.row)).astype(np.float32))
    dec = Decoder(s)
    idx = torch.arange(s.N, dtype=torch.int32, device="cuda").view(1, 1, -1).contiguous()
    dec.decode(bf16(q), bf16(kv), token_idx=idx)
    torch.cuda.synchronize()
    out = to_np(dec.out).reshape(s.G, s.DV)
    lse = to_np(dec.lse).reshape(s.G)
    o_ref, l_ref = oracle.attend_pair(s, q[0], kv[0, 0], np.arange(s.N))
    err = float(np.max(np.abs(out - o_ref)))
    log(f"[gpu] 128-channel attention over every token: max err {err:.2e}")
    assert err <= 2e-3
    assert np.max(np.abs(lse - l_ref)) <= 2e-3


def test_select_all_equals_dense_attention():
    """Kb >= NB and Kt >= N: the GPU step equals dense attention over the whole cache."""
    s = SMALL["select_all"]
    q, kv, lab = inputs(s, seed=5)
    run = GpuRun(s, q, kv, lab)
    gb, _ = run.blocks()
    assert np.all(gb == np.arange(s.NB))
    gt = run.tokens()
    assert np.all(gt[:, : s.N] == np.arange(s.N))
    assert np.all(gt[:, s.N:] == -1)          # Kt' = NB*bs > N: padded after the valid tokens
    out, lse = run.attend()
    for p in range(s.pairs):
        b, h = divmod(p, s.Hkv)
        o_ref, l_ref = oracle.attend_pair(s, q[b, h * s.G:(h + 1) * s.G], kv[b, h], np.arange(s.N))
        assert np.max(np.abs(out[p] - o_ref)) <= 2e-3
        assert np.max(np.abs(lse[p] - l_ref)) <= 2e-3


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_integer_ties_are_broken_by_lower_index(seed):
    """Integer q and K make fp32 scores exact and force many exact ties: the GPU
    sets must then equal the oracle's exactly (lower index wins)."""
    s = W.small_shape(B=2, Hq=8, Hkv=2, N=2048, bs=16, D=64, DV=64, r=4, Kb=37, Kt=150)
    q, kv, lab = inputs(s, int_range=1, seed=seed)
    st = check_all(s, q, kv, lab, expect_exact=True)
    log(f"[gpu] integer ties seed {seed}: {st}")


@pytest.mark.parametrize("keys", ["few_values", "powers_of_two"])
def test_integer_ties_in_wide_rows(keys):
    """Exact ties in rows wide enough for the 1024-thread token selection (4800
    candidates, 1024 first-pass bins). few_values: keys in {-2..2} leave about
    50 distinct scores, so the bins holding the cuts hold hundreds of equal
    keys and the radix passes after the first decide. powers_of_two: keys in
    {0, +-1, +-2, +-4} and q in -6..6 leave 80-200 distinct scores per row;
    the cut bins then hold 29-77 keys of one or a few values, resolved by the
    few-key gather where they are at most 64 and by radix passes elsewhere.
    In both, every label-channel scale is a power of two times 1/7, so equal
    scores are equal in fp32 and in the oracle's fp64 alike, and the sets must
    equal the oracle's exactly (lower index wins)."""
    s = W.small_shape(B=1, Hq=8, Hkv=2, N=16000, bs=16, D=64, DV=64, r=4, Kb=300, Kt=2000)
    if keys == "few_values":
        q, kv, lab = inputs(s, int_range=2, seed=7)
    else:
        rng = np.random.default_rng(11)
        q = W.f32_to_bf16_bits(rng.integers(-6, 7, (s.B, s.Hq, s.D)).astype(np.float32))
        vals = np.array([-4, -2, -1, 0, 1, 2, 4], dtype=np.float32)
        kv = W.f32_to_bf16_bits(rng.choice(vals, (s.B, s.Hkv, s.N, s.row)))
        lab = np.stack([np.sort(rng.choice(s.D, s.r, replace=False)) for _ in range(s.Hkv)]).astype(np.int32)
    st = check_all(s, q, kv, lab, expect_exact=True)
    log(f"[gpu] integer ties, wide rows ({keys}): {st}")


def test_build_exact_ties_round_half_to_even():
    """The label cache built on the GPU for keys whose quotients k / scale are exact
    half-way cases (label absmax 7 * 2^e, so the scale is 2^e): codes round half to
    even (hand-written table), bit-exact with the oracle."""
    import two_level_sparse_amd as T
    from two_level_sparse_amd.runtime import Cache
    half_even = {0.5: 0, 1.5: 2, 2.5: 2, 3.5: 4, 4.5: 4, 5.5: 6, 6.5: 6,
                 -0.5: 0, -1.5: -2, -2.5: -2, -3.5: -4, -4.5: -4, -5.5: -6, -6.5: -6}
    ties = list(half_even)
    lab = np.array([[0, 2, 3, 5, 8, 11, 12, 15]], dtype=np.int32)
    rows, expect = [], []
    for e in (0, -2, 3):
        for part in (ties[:7], ties[7:]):
            a = 7.0 if part[0] > 0 else -7.0
            rows.append([a * 2.0 ** e] + [v * 2.0 ** e for v in part])
            expect.append([7 if a > 0 else -7] + [half_even[v] for v in part])
    s = W.small_shape(B=1, Hq=2, Hkv=1, D=64, DV=64, N=len(rows), bs=4, r=8, Kb=1, Kt=1, n_outlier=0)
    kv = np.zeros((1, 1, s.N, s.row), dtype=np.uint16)
    kv[0, 0][:, lab[0]] = W.f32_to_bf16_bits(np.array(rows, dtype=np.float32))
    cache = Cache(s, kv, lab).build()
    torch.cuda.synchronize()
    codes = to_np(cache.codes).reshape(s.N, s.r // 2)
    ref_codes, ref_scale = oracle.quantize_pair(s, kv[0, 0], lab[0])
    assert ref_codes.tolist() == expect
    np.testing.assert_array_equal(codes, oracle.pack_codes(np.array(expect, dtype=np.int8)))
    np.testing.assert_array_equal(to_np(cache.scale).reshape(-1).view(np.uint32), ref_scale.view(np.uint32))


def test_deterministic():
    s = SMALL["gqa4"]
    q, kv, lab = inputs(s, seed=9)
    run = GpuRun(s, q, kv, lab)
    a = [run.blocks()[0], run.tokens(), run.attend()[0]]
    b = [run.blocks()[0], run.tokens(), run.attend()[0]]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_workspace_too_small_is_rejected():
    import two_level_sparse_amd as T
    s = SMALL["gqa4"]
    q, kv, lab = inputs(s, seed=1)
    run = GpuRun(s, q, kv, lab)
    d = run.dec
    with pytest.raises(T.TlsError) as e:
        T.tls_sparse_decode(d.shape, run.qd, run.cache.kv, None, 0, d.token_idx, d.out, d.lse,
                            d.ws[T.TLS_WS_DECODE], 16)
    assert e.value.code == T.TLS_ERR_WORKSPACE
    with pytest.raises(T.TlsError) as e:
        T.tls_select_blocks(d.shape, run.qd, run.cache.summ, d.block_idx, None, d.ws[T.TLS_WS_BLOCKS], 16)
    assert e.value.code == T.TLS_ERR_WORKSPACE


def test_decode_workspace_counters_return_to_zero_across_shapes():
    """The attention's per-group counters (first 64 KiB of the decode
    workspace) are zero after every call, and calls of different shapes can
    share one workspace: shapes A, B, A on one zero-filled workspace give, bit
    for bit, the outputs of each shape's own workspace."""
    import two_level_sparse_amd as T
    runs = []
    for name, seed in (("gqa4", 5), ("many_splits", 6)):
        s = SMALL[name]
        q, kv, lab = inputs(s, seed=seed)
        run = GpuRun(s, q, kv, lab)
        run.dec.step(run.qd, run.cache)
        torch.cuda.synchronize()
        runs.append((run, to_np(run.dec.out).copy(), to_np(run.dec.lse).copy()))
    size = max(run.dec.ws_sizes[T.TLS_WS_DECODE] for run, _, _ in runs)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for run, ref_out, ref_lse in (runs[0], runs[1], runs[0]):
        d = run.dec
        d.out.zero_(); d.lse.zero_()
        T.tls_sparse_decode(d.shape, run.qd, run.cache.kv, None, 0, d.token_idx, d.out, d.lse, ws, size)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(d.out), ref_out)
        np.testing.assert_array_equal(to_np(d.lse), ref_lse)
        assert not ws[:65536].any().item()


def test_split_merge_reads_this_calls_partials():
    """The split merge inside the 128-channel attention hands the partials from
    workgroup to workgroup (on any XCDs) within the launch: calls on one
    workspace alternating between two queries each give, bit for bit, the
    first output of their query -- a merge that read a partial left by the
    previous call would mix them."""
    from two_level_sparse_amd.runtime import bf16
    s = SMALL["many_splits"]
    q, kv, lab = inputs(s, seed=8)
    run = GpuRun(s, q, kv, lab)
    d = run.dec
    d.step(run.qd, run.cache)
    q2 = bf16(W.gen_q(s.with_(seed=s.seed + 50)))
    torch.cuda.synchronize()
    refs = []
    for qq in (run.qd, q2):
        d.decode(qq, run.cache.kv)
        torch.cuda.synchronize()
        refs.append(to_np(d.out).copy())
    assert np.abs(refs[0] - refs[1]).max() > 1e-3  # the two outputs differ
    for i in range(60):
        d.decode((run.qd, q2)[i % 2], run.cache.kv)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(d.out), refs[i % 2])


def test_graph_replay_matches_eager():
    """The three calls captured in a HIP graph: every replay equals the eager step."""
    s = SMALL["gqa4"]
    q, kv, lab = inputs(s, seed=4)
    run = GpuRun(s, q, kv, lab)
    d = run.dec
    d.step(run.qd, run.cache)
    torch.cuda.synchronize()
    ref = [to_np(d.block_idx), to_np(d.token_idx), to_np(d.out)]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            d.step(run.qd, run.cache)
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        d.out.zero_(); d.token_idx.fill_(-7); d.block_idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(d.block_idx), ref[0])
        np.testing.assert_array_equal(to_np(d.token_idx), ref[1])
        np.testing.assert_array_equal(to_np(d.out), ref[2])


# ------------------------------------------------------- full workloads ---

def full_inputs(s):
    q = W.gen_q(s)
    kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    return q, kv, lab


@pytest.mark.parametrize("name,pairs", [
    ("c1_8k_gqa8", None),
    ("c2_32k_gqa", list(range(0, 32, 2))),
    ("c3_128k_gqa", list(range(0, 64, 4))),
    ("c4_64k_mla", None),
])
def test_full_workloads_sampled(name, pairs):
    """The benchmark's full-size workloads in the launch configuration it uses;
    the oracle checks the sampled (batch, kv-head) pairs."""
    s = W.CONFIGS[name]
    log(f"[gpu] full workload {name}: generating inputs")
    q, kv, lab = full_inputs(s)
    log(f"[gpu] full workload {name}: running")
    st = check_all(s, q, kv, lab, pairs=pairs)
    log(f"[gpu] {name}: {st}")
    del kv
