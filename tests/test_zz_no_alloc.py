"""tls_sparse_decode_noalloc (the attention for callers that cannot allocate:
split partials in the library's own device array) against tls_sparse_decode,
the entry point with a caller workspace, on the same inputs and token sets:
the same kernels, so the outputs must be identical bit for bit. Calls run in a
row on one device -- the full 32k GQA decode, then smaller inputs (a ragged GQA
shape, the latent-attention shape) -- since every call reuses the array the
previous one left behind."""
import numpy as np
import pytest
import torch

import workload as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_level_sparse_amd as T
    T.load_library()


def decode_both(s):
    import two_level_sparse_amd as T
    from two_level_sparse_amd.runtime import Cache, Decoder, bf16
    q = W.gen_q(s)
    kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    cache = Cache(s, kv, lab).build()
    dec = Decoder(s)
    qd = bf16(q)
    dec.select(qd, cache)
    out = torch.full_like(dec.out, float("nan"))
    lse = torch.full_like(dec.lse, float("nan"))
    torch.cuda.synchronize()
    print(f"[gpu] noalloc: {s.name} B={s.B} Hq={s.Hq} Hkv={s.Hkv} D={s.D} N={s.N} Kt={s.Kt}", flush=True)
    T.tls_sparse_decode_noalloc(dec.shape, qd, cache.kv, None, 0, dec.token_idx, out, lse)
    dec.decode(qd, cache.kv)  # the entry point with a workspace
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), dec.out.cpu().numpy(), dec.lse.cpu().numpy()


def test_noalloc_decode_matches_the_workspace_entry_point_on_calls_in_a_row():
    import two_level_sparse_amd as T
    shapes = [W.CONFIGS["c2_32k_gqa"],
              W.small_shape(name="gqa8_ragged", B=2, Hq=16, Hkv=2, N=1000, bs=64, Kb=5, Kt=200),
              W.small_shape(name="mla_small", B=2, Hq=128, Hkv=1, D=576, DV=512, v_is_k_prefix=True, N=2048,
                            bs=64, r=32, Kb=8, Kt=300)]
    sizes = [T.tls_workspace_size(T.shape_of(s), T.TLS_WS_DECODE) for s in shapes]
    assert sizes[1] < sizes[0]  # the second call writes less of the array than the first
    assert all(0 < n <= T.TLS_NOALLOC_SCRATCH_BYTES for n in sizes)
    for s in shapes:
        out, lse, out_ref, lse_ref = decode_both(s)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
        np.testing.assert_array_equal(out, out_ref)
        np.testing.assert_array_equal(lse, lse_ref)
