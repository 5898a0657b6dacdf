"""The C ABI library loads, exports every function include/csa2.h declares,
and rejects invalid arguments on the host before launching anything (these
calls never reach a kernel, so they run without a GPU)."""
import ctypes
import subprocess
import threading

import pytest

from sparse_attention_decode_e2m1_amd import api

FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def L():
    return api.lib()


def test_exports_every_declared_symbol(L):
    names = api.declared_functions()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert getattr(L, n) is not None


def test_struct_layout(L):
    assert L.csa2_layer_args_size() == ctypes.sizeof(api.LayerArgs)
    assert L.csa2_fp4_cache_size() == ctypes.sizeof(api.Fp4Cache)


def test_bytes_per_token(L):
    assert L.csa2_fp4_bytes_per_token(576) == 324
    assert L.csa2_fp4_bytes_per_token(128) == 72
    assert L.csa2_fp4_bytes_per_token(15) == -1


def test_status_strings(L):
    for s in range(8):
        assert L.csa2_status_string(s)
    assert b"gave up" in L.csa2_status_string(api.ERR_INCOMPLETE)
    assert L.csa2_status_string(99) == b"unknown status"
    assert b"gfx950" in L.csa2_version()


def test_quantize_rejects(L):
    q = L.csa2_quantize_kv
    assert q(FAKE, 7, 4, 576, 576, None, FAKE, FAKE, None) == 3          # dtype
    assert q(FAKE, 0, 4, 100, 100, None, FAKE, FAKE, None) == 2          # dim % 16
    assert q(FAKE, 0, 4, 576, 500, None, FAKE, FAKE, None) == 2          # stride < dim
    assert q(FAKE, 0, -1, 576, 576, None, FAKE, FAKE, None) == 2         # rows < 0
    assert q(None, 0, 4, 576, 576, None, FAKE, FAKE, None) == 1          # null x
    assert b"required" in L.csa2_last_error()
    assert q(None, 0, 0, 576, 576, None, None, None, None) == 0          # nothing to do


def test_rope_quantize_rejects(L):
    q = L.csa2_rope_quantize_kv
    assert q(FAKE, 7, 4, 576, 576, 64, FAKE, None, FAKE, FAKE, None) == 3   # dtype
    assert q(FAKE, 0, 4, 576, 576, 60, FAKE, None, FAKE, FAKE, None) == 2   # rope_dim % 16
    assert q(FAKE, 0, 4, 576, 576, 592, FAKE, None, FAKE, FAKE, None) == 2  # rope_dim > dim
    assert q(FAKE, 0, 4, 576, 576, 64, None, None, FAKE, FAKE, None) == 1   # cos_sin missing
    assert b"cos_sin" in L.csa2_last_error()
    assert q(FAKE, 0, 0, 576, 576, 64, None, None, None, None, None) == 0   # nothing to do


def test_index_score_rejects(L):
    c = api.Fp4Cache(FAKE, FAKE, 100, 16)
    f = L.csa2_index_score
    assert f(ctypes.byref(c), 1, 1, FAKE, FAKE, 4, FAKE, None, 0, 16, FAKE, None) == 5
    c.dim = 128
    assert f(ctypes.byref(c), 1, 1, FAKE, FAKE, 17, FAKE, None, 0, 16, FAKE, None) == 2
    assert f(ctypes.byref(c), 1, 1, None, FAKE, 4, FAKE, None, 0, 16, FAKE, None) == 1
    assert f(ctypes.byref(c), 1, 1, FAKE, FAKE, 4, FAKE, FAKE, 0, 16, FAKE, None) == 2
    assert f(None, 1, 1, FAKE, FAKE, 4, FAKE, None, 0, 16, FAKE, None) == 1


def test_topk_rejects(L):
    f = L.csa2_topk
    need = L.csa2_topk_workspace_bytes(2, 1000, 10)
    assert need > 0
    assert f(FAKE, 2, 1000, FAKE, None, 0, FAKE, None, FAKE, need, None) == 2       # k < 1
    assert f(FAKE, 2, 1000, FAKE, None, 16385, FAKE, None, FAKE, 1 << 30, None) == 2
    assert f(FAKE, 0, 1000, FAKE, None, 10, FAKE, None, FAKE, need, None) == 2
    assert f(FAKE, 2, 1000, FAKE, None, 10, FAKE, None, FAKE, need - 1, None) == 4  # workspace
    assert b"workspace" in L.csa2_last_error()
    assert f(FAKE, 2, 1000, FAKE, None, 10, FAKE, None, None, need, None) == 4
    assert f(None, 2, 1000, FAKE, None, 10, FAKE, None, FAKE, need, None) == 1


def test_sparse_attn_rejects(L):
    kv = api.Fp4Cache(FAKE, FAKE, 576, 100)
    f = L.csa2_sparse_attn
    need = L.csa2_sparse_attn_workspace_bytes(1, 64, 128, 512)
    args = lambda H=16, dv=512, K=64, ws=FAKE, nb=need: (
        FAKE, 1, 1, H, ctypes.byref(kv), FAKE, K, FAKE, FAKE, FAKE, 128, 128, FAKE,
        ctypes.c_float(0.04), dv, FAKE, None, ws, nb, None)
    for f in (L.csa2_sparse_attn, L.csa2_sparse_attn_one_launch):
        assert f(*args(H=8)) == 5
        assert f(*args(dv=256)) == 5
        assert f(*args(K=-1)) == 2
        assert f(*args(nb=need - 1)) == 4
        assert f(*args(ws=None)) == 4


def test_fp8_entry_points_reject(L):
    q = L.csa2_quantize_kv_fp8
    assert q(FAKE, 7, 4, 576, 576, None, FAKE, FAKE, None) == 3    # dtype
    assert q(FAKE, 0, 4, 570, 576, None, FAKE, FAKE, None) == 2    # dim % 16
    assert q(FAKE, 0, 4, 576, 500, None, FAKE, FAKE, None) == 2    # stride < dim
    assert q(FAKE, 0, 4, 576, 576, None, FAKE, None, None) == 1    # scales missing
    assert q(None, 0, 0, 576, 576, None, None, None, None) == 0    # nothing to do
    kv = api.Fp8Cache(FAKE, FAKE, 576, 100)
    f = L.csa2_sparse_attn_fp8
    need = L.csa2_sparse_attn_workspace_bytes(1, 64, 128, 512)
    args = lambda H=16, dv=512, K=64, ws=FAKE, nb=need, c=ctypes.byref(kv): (
        FAKE, 1, 1, H, c, FAKE, K, FAKE, FAKE, FAKE, 128, 128, FAKE,
        ctypes.c_float(0.04), dv, FAKE, None, ws, nb, None)
    assert f(*args(c=None)) == 1
    assert f(*args(H=8)) == 5
    assert f(*args(dv=256)) == 5
    assert f(*args(K=-1)) == 2
    assert f(*args(nb=need - 1)) == 4
    assert f(*args(ws=None)) == 4
    kv.scales = None
    assert f(*args()) == 1


def test_layer_step_rejects(L):
    assert L.csa2_layer_step(0, None, FAKE, 1 << 20, None) == 1
    a = api.LayerArgs(B=1, T=1, H=16, D=576, dv=512, H_I=4, D_I=128, K=64, S=128, W=128)
    a.kv = api.Fp4Cache(FAKE, FAKE, 576, 100)
    a.icache = api.Fp4Cache(FAKE, FAKE, 128, 100)
    for name in ("q", "q_pos", "swa", "swa_scale", "swa_pos0", "out", "idx_out", "q_idx", "w_idx",
                 "new_kv", "new_ikey", "idx_in"):
        setattr(a, name, FAKE)
    assert L.csa2_layer_step(9, ctypes.byref(a), FAKE, 1 << 30, None) == 2     # unknown mode
    need = L.csa2_workspace_bytes(0, ctypes.byref(a))
    assert need > 0
    assert L.csa2_layer_step(0, ctypes.byref(a), FAKE, need - 1, None) == 4
    a.new_kv = None
    assert L.csa2_layer_step(0, ctypes.byref(a), FAKE, need, None) == 1       # FULL needs rows
    a.new_kv = FAKE
    a.P = 8                                                                 # P < K
    assert L.csa2_layer_step(0, ctypes.byref(a), FAKE, 1 << 30, None) == 2
    a.P = 0
    a.new_dtype = 5
    assert L.csa2_layer_step(0, ctypes.byref(a), FAKE, 1 << 30, None) == 3
    a.new_dtype = 0
    a.D_I = 64
    a.icache = api.Fp4Cache(FAKE, FAKE, 64, 100)
    assert L.csa2_layer_step(1, ctypes.byref(a), FAKE, 1 << 30, None) == 5
    # REUSE needs no index cache
    a.icache = api.Fp4Cache(None, None, 0, 0)
    assert L.csa2_workspace_bytes(2, ctypes.byref(a)) > 0


def test_workspace_check_rejects(L):
    """csa2_workspace_check validates before touching the device."""
    f = L.csa2_workspace_check
    ctl = L.csa2_workspace_control_bytes(4)
    assert ctl > 0
    assert f(None, ctl, 4, None) == 1                 # no workspace
    assert f(FAKE, ctl, 0, None) == 2                 # rows < 1
    assert f(FAKE, ctl - 1, 4, None) == 4             # smaller than the control block
    assert b"control bytes" in L.csa2_last_error()
    # the control block covers at most one pass of 256 rows
    assert L.csa2_workspace_control_bytes(10_000) == L.csa2_workspace_control_bytes(256)


def test_topk_variant_and_wait_limit_controls(L):
    """The diagnostic setters return the previous value; an unknown variant
    falls back to automatic choice."""
    try:
        assert api.set_topk_variant(api.TOPK_SELECT_CUT) == api.TOPK_AUTO
        assert api.set_topk_variant(api.TOPK_ROW) == api.TOPK_SELECT_CUT
        assert api.set_topk_variant(42) == api.TOPK_ROW
        assert api.set_topk_variant(api.TOPK_AUTO) == api.TOPK_AUTO   # 42 was stored as AUTO
        assert api.set_topk_variant(-3) == api.TOPK_AUTO
        assert api.set_topk_variant(api.TOPK_SAMPLED_FALLBACK) == api.TOPK_AUTO
        assert api.set_topk_variant(api.TOPK_BAND) == api.TOPK_SAMPLED_FALLBACK
        assert api.set_topk_variant(api.TOPK_BAND_EXACT) == api.TOPK_BAND
        assert api.set_topk_variant(api.TOPK_BAND_EXACT + 1) == api.TOPK_BAND_EXACT
        assert api.set_topk_variant(api.TOPK_AUTO) == api.TOPK_AUTO   # one past the last: AUTO
    finally:
        api.set_topk_variant(api.TOPK_AUTO)
    try:
        assert api.set_wait_limit(0) == 1 << 20
        assert api.set_wait_limit(123) == 0
    finally:
        api.set_wait_limit(1 << 20)
    # per host thread: a thread that ran no Top-K pass reads -1 (a fresh
    # thread, since GPU tests earlier in the same process may have run some)
    seen = []
    th = threading.Thread(target=lambda: seen.append(api.topk_last_variant()))
    th.start()
    th.join()
    assert seen == [-1]
