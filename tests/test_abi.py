"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol include/tls.h declares, sizes workspaces, and rejects bad arguments
before touching the device."""
import ctypes as C
import re
from pathlib import Path

import pytest

import two_level_sparse_amd as T
import workload as W

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def lib():
    if not T.LIB_PATH.exists():
        from two_level_sparse_amd import build
        build.build()
    return T.load_library()


def declared_functions():
    hdr = (ROOT / "include" / "tls.h").read_text()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    return sorted(set(re.findall(r"\b(tls_[a-z_0-9]+)\s*\(", hdr)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    raw = C.CDLL(str(T.LIB_PATH))
    for n in names:
        assert hasattr(raw, n), n
    assert sorted(T.EXPORTED) == names
    assert T.tls_version().startswith("tls-gfx950")


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_workspace_sizes(lib, name):
    s = W.CONFIGS[name]
    sh = T.shape_of(s)
    assert T.tls_workspace_size(sh, T.TLS_WS_BLOCKS) >= s.pairs * s.NB * 4
    assert T.tls_workspace_size(sh, T.TLS_WS_TOKENS) > 0
    dec = T.tls_workspace_size(sh, T.TLS_WS_DECODE)
    assert dec >= s.Hq * s.B * (s.DV + 2) * 4
    assert T.tls_workspace_size(sh, 7) == 0
    step = T.tls_workspace_size(sh, T.TLS_WS_STEP)
    if s.D == 128 and not s.v_is_k_prefix and s.G <= 8:
        # the one-launch step: state words, block scores and the partials
        assert step >= s.pairs * s.NB * 4 + s.pairs * ((s.Kt + 255) // 256) * 8 * 132 * 4
    else:
        assert step == 0   # shapes it does not cover (the 64k latent-attention workload)


def test_one_launch_step_rejects_what_it_does_not_cover(lib):
    s = W.CONFIGS["c4_64k_mla"]
    rc = lib.tls_decode_step(C.byref(T.shape_of(s)), 16, 16, 16, 16, 16, 16, 16, 16, 16, None, 256, 1 << 30, None)
    assert rc == T.TLS_ERR_UNSUPPORTED
    s = W.CONFIGS["c3_128k_gqa"]
    sh = T.shape_of(s)
    rc = lib.tls_decode_step(C.byref(sh), 16, 16, 16, 16, 16, 16, 16, 16, 16, None, 256, 16, None)
    assert rc == T.TLS_ERR_WORKSPACE
    rc = lib.tls_decode_step(C.byref(sh), 16, 16, 16, 16, 16, None, 16, 16, 16, None, 256, 1 << 30, None)
    assert rc == T.TLS_ERR_INVALID_ARG
    for bad in (dict(Hq=128), dict(bs=32), dict(r=32), dict(Kb=200)):
        assert T.tls_workspace_size(T.shape_of(s.with_(**bad)), T.TLS_WS_STEP) == 0, bad


def test_invalid_shapes_give_zero_workspace(lib):
    s = W.CONFIGS["c2_32k_gqa"]
    for bad in (dict(Hq=30), dict(N=0), dict(bs=0), dict(r=3), dict(Kb=0), dict(Kt=0)):
        assert T.tls_workspace_size(T.shape_of(s.with_(**bad)), T.TLS_WS_BLOCKS) == 0, bad
    # valid but not compiled: bs > 64, G > 128
    assert T.tls_workspace_size(T.shape_of(s.with_(bs=128)), T.TLS_WS_BLOCKS) == 0
    assert T.tls_workspace_size(T.shape_of(s.with_(Hq=8 * 256)), T.TLS_WS_BLOCKS) == 0


def test_argument_errors_before_any_device_work(lib):
    s = W.CONFIGS["c1_8k_gqa8"]
    sh = T.shape_of(s)
    rc = lib.tls_select_blocks(C.byref(sh), None, None, None, None, None, 0, None)
    assert rc == T.TLS_ERR_INVALID_ARG and b"NULL" in lib.tls_last_error()
    rc = lib.tls_select_blocks(C.byref(sh), 16, 16, 16, None, 16, 8, None)
    assert rc == T.TLS_ERR_WORKSPACE
    rc = lib.tls_sparse_decode(C.byref(sh), 16, 16, None, 0, 16, 16, None, 16, 8, None)
    assert rc == T.TLS_ERR_WORKSPACE
    rc = lib.tls_select_tokens(C.byref(sh), 16, 16, None, 16, 16, 16, None, 0, None)
    assert rc == T.TLS_ERR_INVALID_ARG
    rc = lib.tls_sparse_decode(C.byref(T.shape_of(s.with_(D=96, DV=96))), 16, 16, None, 0, 16, 16, None, 16, 1 << 30,
                               None)
    assert rc == T.TLS_ERR_UNSUPPORTED
    rc = lib.tls_sparse_decode(C.byref(sh), 8, 16, None, 0, 16, 16, None, 16, 1 << 30, None)
    assert rc == T.TLS_ERR_INVALID_ARG   # q not 16-byte aligned
    rc = lib.tls_select_blocks(None, 16, 16, 16, None, 16, 1 << 30, None)
    assert rc == T.TLS_ERR_INVALID_ARG
    h = C.c_void_p()
    rc = lib.tls_offload_create(C.byref(sh), None, None, None, None, None, C.byref(h))
    assert rc == T.TLS_ERR_INVALID_ARG and h.value is None
    rc = lib.tls_prefetch_delta(None, 0, None, None, None, None)
    assert rc == T.TLS_ERR_INVALID_ARG
    # the measurement hook takes both events or neither, for a known kernel
    rc = lib.tls_profile_events(T.TLS_PROFILE_ATTENTION, 16, None)
    assert rc == T.TLS_ERR_INVALID_ARG and b"both" in lib.tls_last_error()
    assert lib.tls_profile_events(7, None, None) == T.TLS_ERR_INVALID_ARG
    assert lib.tls_profile_events(T.TLS_PROFILE_BLOCK_SCORES, None, None) == T.TLS_OK


def test_noalloc_decode_checks_before_any_device_work(lib):
    """tls_sparse_decode_noalloc: NULL buffers, and shapes whose split partials
    exceed its device array, are refused before the array is looked up; every
    workload here fits the array."""
    sh = T.shape_of(W.CONFIGS["c1_8k_gqa8"])
    assert lib.tls_sparse_decode_noalloc(C.byref(sh), None, 16, None, 0, 16, 16, None, None) == T.TLS_ERR_INVALID_ARG
    for name, s in W.CONFIGS.items():
        assert 0 < T.tls_workspace_size(T.shape_of(s), T.TLS_WS_DECODE) <= T.TLS_NOALLOC_SCRATCH_BYTES, name
    big = W.CONFIGS["c4_64k_mla"].with_(B=64)
    assert T.tls_workspace_size(T.shape_of(big), T.TLS_WS_DECODE) > T.TLS_NOALLOC_SCRATCH_BYTES
    rc = lib.tls_sparse_decode_noalloc(C.byref(T.shape_of(big)), 16, 16, None, 0, 16, 16, None, None)
    assert rc == T.TLS_ERR_WORKSPACE and b"scratch array" in lib.tls_last_error()


def test_select_both_stages_arguments_and_workspace(lib):
    """tls_select (both selection stages in one call): its workspace holds the
    block scores and the token stage's workspace; it rejects what either
    stage rejects, before any device work."""
    for name in W.CONFIGS:
        sh = T.shape_of(W.CONFIGS[name])
        blocks = lib.tls_workspace_size(C.byref(sh), T.TLS_WS_BLOCKS)
        tokens = lib.tls_workspace_size(C.byref(sh), T.TLS_WS_TOKENS)
        sel = lib.tls_workspace_size(C.byref(sh), T.TLS_WS_SELECT)
        assert sel >= blocks + tokens > 0, name
    s = W.CONFIGS["c1_8k_gqa8"]
    sh = T.shape_of(s)
    rc = lib.tls_select(C.byref(sh), 16, 16, 16, 16, 16, None, 16, 16, 1 << 30, None)
    assert rc == T.TLS_ERR_INVALID_ARG and b"NULL" in lib.tls_last_error()
    rc = lib.tls_select(C.byref(sh), 16, 16, 16, 16, 16, 16, 16, 256, 8, None)
    assert rc == T.TLS_ERR_WORKSPACE
    rc = lib.tls_select(C.byref(sh), 8, 16, 16, 16, 16, 16, 16, 256, 1 << 30, None)
    assert rc == T.TLS_ERR_INVALID_ARG   # q not 16-byte aligned
    # more candidates than the token stage takes: no workspace size, and the call says why
    big = T.shape_of(W.CONFIGS["c3_128k_gqa"].with_(Kb=2048, Kt=131072))
    assert lib.tls_workspace_size(C.byref(big), T.TLS_WS_SELECT) == 0
    rc = lib.tls_select(C.byref(big), 16, 16, 16, 16, 16, 16, 16, 256, 1 << 30, None)
    assert rc == T.TLS_ERR_UNSUPPORTED and b"candidate" in lib.tls_last_error()


def test_candidate_limit_applies_to_the_token_stage_only(lib):
    """Attention over every token (Kb >= NB, Kt >= N) is a valid decode shape even
    when Kb*bs exceeds what the token stage takes (16384 candidates per pair)."""
    s = W.CONFIGS["c3_128k_gqa"].with_(Kb=2048, Kt=131072)
    sh = T.shape_of(s)
    assert lib.tls_workspace_size(C.byref(sh), T.TLS_WS_TOKENS) == 0
    assert lib.tls_workspace_size(C.byref(sh), T.TLS_WS_DECODE) > 0
    assert lib.tls_workspace_size(C.byref(sh), T.TLS_WS_BLOCKS) > 0
    rc = lib.tls_select_tokens(C.byref(sh), 16, 16, 16, 16, 16, 16, 16, 1 << 30, None)
    assert rc == T.TLS_ERR_UNSUPPORTED and b"candidate" in lib.tls_last_error()


def test_token_selection_over_the_whole_cache_takes_passes(lib):
    """Kb >= NB with Kt' <= 8192 (DS-style selection over every token): the token
    stage selects in passes over chunks of 16384 candidates, with room for the
    scores and two (key, id) lists in its workspace."""
    s = W.CONFIGS["c3_128k_gqa"].with_(Kb=2048)        # 131072 candidates, Kt = 4096
    ws = lib.tls_workspace_size(C.byref(T.shape_of(s)), T.TLS_WS_TOKENS)
    scores = s.pairs * s.N * 4
    lists = s.pairs * (s.N // 16384) * s.Kt * 4
    assert ws >= scores + 4 * lists
    too_many = s.with_(Kt=8193)
    assert lib.tls_workspace_size(C.byref(T.shape_of(too_many)), T.TLS_WS_TOKENS) == 0
    within = W.CONFIGS["c3_128k_gqa"].with_(Kb=256, Kt=16384)  # 16384 candidates: one pass, any Kt
    assert lib.tls_workspace_size(C.byref(T.shape_of(within)), T.TLS_WS_TOKENS) == within.pairs * 16384 * 4


def test_append_checks_the_capacity_before_any_device_work(lib):
    """tls_append_kv: the grown length must fit the allocated capacity, which
    must itself hold the current length; an offload context takes a capacity
    of whole blocks, with at least Kb blocks present when it is to grow."""
    s = W.small_shape(N=1000)
    sh = T.shape_of(s, capacity=1064)
    rc = lib.tls_append_kv(C.byref(sh), None, 1, 16, 16, 16, 16, 16, None)
    assert rc == T.TLS_ERR_INVALID_ARG and b"NULL" in lib.tls_last_error()
    rc = lib.tls_append_kv(C.byref(sh), 16, 0, 16, 16, 16, 16, 16, None)
    assert rc == T.TLS_ERR_INVALID_ARG and b"n_new" in lib.tls_last_error()
    rc = lib.tls_append_kv(C.byref(sh), 16, 65, 16, 16, 16, 16, 16, None)
    assert rc == T.TLS_ERR_INVALID_ARG and b"capacity" in lib.tls_last_error()
    rc = lib.tls_append_kv(C.byref(sh), 8, 1, 16, 16, 16, 16, 16, None)
    assert rc == T.TLS_ERR_INVALID_ARG   # new_kv not 16-byte aligned
    small = T.shape_of(s, capacity=999)
    assert lib.tls_workspace_size(C.byref(small), T.TLS_WS_BLOCKS) == 0
    rc = lib.tls_append_kv(C.byref(small), 16, 1, 16, 16, 16, 16, 16, None)
    assert rc == T.TLS_ERR_INVALID_ARG and b"ctx_capacity" in lib.tls_last_error()
    # a capacity beyond the length is a valid shape for every call
    assert lib.tls_workspace_size(C.byref(sh), T.TLS_WS_DECODE) > 0
    # offloaded caches: whole blocks of capacity, and a growing one needs Kb blocks from the start
    h = C.c_void_p()
    off = T.shape_of(s.with_(N=1024), capacity=1090)
    rc = lib.tls_offload_create(C.byref(off), 16, 16, 16, 16, 16, C.byref(h))
    assert rc == T.TLS_ERR_UNSUPPORTED and h.value is None and b"multiple" in lib.tls_last_error()
    few = T.shape_of(s.with_(N=64 * (s.Kb - 1), Kb=s.Kb), capacity=64 * (s.Kb + 4))
    rc = lib.tls_offload_create(C.byref(few), 16, 16, 16, 16, 16, C.byref(h))
    assert rc == T.TLS_ERR_UNSUPPORTED and h.value is None and b"top_kb" in lib.tls_last_error()
    rc = lib.tls_offload_append(None, 16, 1, 16, 16, 16, 16, None)
    assert rc == T.TLS_ERR_INVALID_ARG
