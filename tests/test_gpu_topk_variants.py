"""Every Top-K variant the dispatcher can choose, forced through
csa2_set_topk_variant and named in the test id, bit-exact against the
oracle's selection on the same fp32 scores (order: score descending, the
lower slot first among equal scores, -0 == +0; output ascending, -1 padded).
Each case also checks which variant actually ran (csa2_topk_last_variant),
so a case cannot pass on another variant by accident of occupancy.

The one-wait variant's failure path is forced from the host: a wait limit of
0 makes every block that would wait for its record give up at once (every
kernel still exits normally).  csa2_workspace_check must then report
CSA2_ERR_INCOMPLETE, and later calls on the same workspace must be correct
whether or not the check ran in between."""
import functools

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_e2m1_amd import api
from tests.gpu_common import dev, host

pytestmark = pytest.mark.gpu

BITMAP_N = 200_003          # rows finished from a bitmap (<= 2^19 slots)
LIST_N = (1 << 20) + 13     # rows finished by merging sorted lists (> 2^19 slots)


@pytest.fixture(autouse=True)
def _auto_after():
    yield
    api.set_topk_variant(api.TOPK_AUTO)
    api.set_wait_limit(1 << 20)


_KIND_SEED = {"normal": 0, "ties": 1, "salient": 2}


@functools.lru_cache(maxsize=None)
def _scores(rows, n, seed, kind):
    rng = np.random.default_rng(seed * 10 + _KIND_SEED[kind])
    if kind == "normal":
        s = rng.standard_normal((rows, n))
    elif kind == "ties":
        s = np.round(rng.standard_normal((rows, n)), 1)
        s[-1] = np.where(rng.random(n) < 0.5, -0.0, 0.0)  # one tie storm of signed zeros
    else:  # "salient": a few large scores above a dense bulk (the pool workload's shape)
        s = rng.standard_normal((rows, n))
        hot = rng.choice(n, max(1, n // 100), replace=False)
        s[:, hot] += 8.0
    return s.astype(np.float32)  # cached: callers never write to it


def _run(scores, nv, k, slot_pos=None, ws=None):
    rows, n = scores.shape
    if ws is None:
        ws = api.workspace(api.topk_workspace_bytes(rows, n, k))
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    api.topk(dev(scores), dev(np.asarray(nv, np.int32)), k, idx, ws,
             slot_pos=None if slot_pos is None else dev(slot_pos), count_out=cnt)
    torch.cuda.synchronize()
    return host(idx), host(cnt), ws


_EXPECT = {}


def _expect(scores, nv, k, slot_pos=None):
    key = (id(scores), scores.shape, tuple(np.asarray(nv).tolist()), k,
           None if slot_pos is None else id(slot_pos))
    if key not in _EXPECT:
        _EXPECT[key] = _expect_now(scores, nv, k, slot_pos)
    return _EXPECT[key]


def _expect_now(scores, nv, k, slot_pos=None):
    out = []
    for r in range(scores.shape[0]):
        sp = None if slot_pos is None else slot_pos[r]
        o, c = oracle.topk(scores[r].astype(np.float64), int(nv[r]), k, slot_pos=sp)
        out.append((o, c))
    return out


def _check(scores, nv, k, want_variant, slot_pos=None):
    g, cnt, ws = _run(scores, nv, k, slot_pos)
    assert api.topk_last_variant() == want_variant, (api.topk_last_variant(), want_variant)
    for r, (o, c) in enumerate(_expect(scores, nv, k, slot_pos)):
        assert np.array_equal(g[r], o), (r, k, int(nv[r]))
        assert cnt[r] == c, (r, cnt[r], c)
    words = ws[: api.lib().csa2_workspace_control_bytes(scores.shape[0])].view(torch.int32)
    assert int(torch.count_nonzero(words)) == 0, "control words not cleared"
    api.workspace_check(ws, scores.shape[0])


SELECT_VARIANTS = [("select", api.TOPK_SELECT), ("select_cut", api.TOPK_SELECT_CUT),
                   ("select_large", api.TOPK_SELECT_LARGE),
                   ("select_large_cut", api.TOPK_SELECT_LARGE_CUT)]


@pytest.mark.parametrize("name,variant", SELECT_VARIANTS, ids=[v[0] for v in SELECT_VARIANTS])
@pytest.mark.parametrize("n,finish", [(BITMAP_N, 0), (LIST_N, api.TOPK_LIST_FINISH)],
                         ids=["bitmap_finish", "list_merge_finish"])
@pytest.mark.parametrize("kind", ["normal", "ties", "salient"])
def test_select_variants(name, variant, n, finish, kind):
    rows = 4 if n == LIST_N else 3
    s = _scores(rows, n, 60 + rows, kind)
    nv = np.full(rows, n, np.int32)
    nv[0] = n - 4095                    # a partial last block
    api.set_topk_variant(variant)
    for k in (2048, 16384):
        _check(s, nv, k, variant | finish)


@pytest.mark.parametrize("kind", ["normal", "ties", "salient"])
def test_one_wait_variant(kind):
    rows, n = 4, (1 << 18)              # 64 blocks a row: 256 resident blocks
    s = _scores(rows, n, 71, kind)
    nv = np.array([n, n - 1, n - 4097, 3000], np.int32)
    api.set_topk_variant(api.TOPK_ONE_WAIT)
    for k in (1, 2048, 16384):
        _check(s, nv, k, api.TOPK_ONE_WAIT)


@pytest.mark.parametrize("kind", ["normal", "ties", "salient"])
def test_row_variant(kind):
    """One block per row at a row count below the automatic threshold (the
    variant serves rows of up to 2^18 slots)."""
    rows, n = 3, (1 << 18)
    s = _scores(rows, n, 72, kind)
    nv = np.array([n, 70000, 2049], np.int32)
    api.set_topk_variant(api.TOPK_ROW)
    for k in (1, 2048, 16384):
        _check(s, nv, k, api.TOPK_ROW)


BAND_SHAPES = [  # (n, visible slots per row): 16 / 8 / 4 keys per thread, partial rows
    (16384, (16384, 16383, 9000, 2049)),
    (12000, (12000, 11999, 5000, 1025)),
    (8192, (8192, 4097, 3000, 300)),
    (4096, (4096, 4095, 1000, 100)),
]


@pytest.mark.parametrize("name,variant", [("band", api.TOPK_BAND),
                                          ("band_exact", api.TOPK_BAND_EXACT)],
                         ids=["band", "band_exact"])
@pytest.mark.parametrize("n,nvs", BAND_SHAPES, ids=[str(b[0]) for b in BAND_SHAPES])
@pytest.mark.parametrize("kind", ["normal", "ties", "salient"])
def test_band_variant(name, variant, n, nvs, kind):
    """One block per row of up to 2^14 slots with a sampled key band, and the
    same block's exact path (forced): K from 1 to past the visible count."""
    s = _scores(len(nvs), n, 80 + n % 97, kind)
    nv = np.array(nvs, np.int32)
    api.set_topk_variant(variant)
    for k in (1, 33, 256, 2048, 3500, 16384):
        _check(s, nv, k, variant)


def test_band_is_the_automatic_choice_for_short_rows():
    s = _scores(2, 16384, 81, "salient")
    nv = np.array([16384, 7000], np.int32)
    _check(s, nv, 2048, api.TOPK_BAND)
    s = _scores(1, 4096, 82, "normal")
    _check(s, np.array([4096], np.int32), 256, api.TOPK_BAND)


@functools.lru_cache(maxsize=None)
def _pool_scores():
    rng = np.random.default_rng(83)
    top = np.sort(rng.standard_normal(1 << 20).astype(np.float32))[-16384:]
    return np.stack([rng.permutation(top), rng.permutation(top)])  # cached: never written


def test_band_needs_rows_of_whole_16_byte_words():
    """A row stride that is not a multiple of 4 slots cannot take the key
    band's 16-byte loads: the automatic choice is the row kernel, same result."""
    s = _scores(2, 4099, 84, "normal")
    nv = np.array([4099, 3001], np.int32)
    _check(s, nv, 256, api.TOPK_ROW)


def test_band_narrow_pool_scores():
    """A pool's scores: the top 16384 of a million, so every key shares its
    leading bits (the sample's own key range sets the bins)."""
    rows = _pool_scores()
    nv = np.array([16384, 16000], np.int32)
    api.set_topk_variant(api.TOPK_BAND)
    for k in (1, 2048, 8000):
        _check(rows, nv, k, api.TOPK_BAND)


def test_forced_variant_that_cannot_serve_falls_back():
    """ROW cannot take rows over 2^18 slots; the pass keeps its own choice."""
    s = _scores(2, 300_000, 73, "normal")
    nv = np.full(2, 300_000, np.int32)
    api.set_topk_variant(api.TOPK_ROW)
    g, _, _ = _run(s, nv, 2048)
    assert api.topk_last_variant() != api.TOPK_ROW
    for r, (o, _) in enumerate(_expect(s, nv, 2048)):
        assert np.array_equal(g[r], o)


def test_slot_map_on_every_variant():
    rng = np.random.default_rng(74)
    P = 16384
    pool = np.stack([np.sort(rng.choice(1 << 20, P, replace=False)) for _ in range(2)]).astype(np.int32)
    s = _scores(2, P, 75, "salient")
    nv = np.array([P, 9000], np.int32)
    for name, v in [("row", api.TOPK_ROW), ("one_wait", api.TOPK_ONE_WAIT), ("band", api.TOPK_BAND),
                    ("band_exact", api.TOPK_BAND_EXACT)] + SELECT_VARIANTS:
        api.set_topk_variant(v)
        _check(s, nv, 2048, v, slot_pos=pool)


def test_one_wait_gave_up_is_reported_and_leaves_no_stale_state():
    """Wait limit 0: every block but the row's completing one gives up.  The
    check reports it; a later call is correct with or without a check in
    between (records carry the launch's generation)."""
    rows, n, k = 4, (1 << 18), 2048
    s = _scores(rows, n, 76, "normal")
    nv = np.full(rows, n, np.int32)
    want = _expect(s, nv, k)
    api.set_topk_variant(api.TOPK_ONE_WAIT)
    api.set_wait_limit(0)
    _, _, ws = _run(s, nv, k)
    assert api.topk_last_variant() == api.TOPK_ONE_WAIT
    api.set_wait_limit(1 << 20)
    with pytest.raises(api.Csa2Error) as e:
        api.workspace_check(ws, rows)
    assert e.value.status == api.ERR_INCOMPLETE
    api.workspace_check(ws, rows)     # the check cleared the flags
    g, _, _ = _run(s, nv, k, ws=ws)
    for r, (o, _) in enumerate(want):
        assert np.array_equal(g[r], o)
    # fail again, then run correctly WITHOUT a check in between
    api.set_wait_limit(0)
    _run(s, nv, k, ws=ws)
    api.set_wait_limit(1 << 20)
    g, _, _ = _run(s, nv, k, ws=ws)
    for r, (o, _) in enumerate(want):
        assert np.array_equal(g[r], o)
    with pytest.raises(api.Csa2Error) as e:
        api.workspace_check(ws, rows)    # the earlier failure is still reported
    assert e.value.status == api.ERR_INCOMPLETE
    words = ws[: api.lib().csa2_workspace_control_bytes(rows)].view(torch.int32)
    assert int(torch.count_nonzero(words)) == 0


def test_one_launch_attention_gave_up_is_reported():
    """The one-launch attention's bounded wait, forced to give up: reported by
    the check; the next call equals the split + merge attention bit for bit."""
    rng = np.random.default_rng(77)
    B, N, K, S, W, D = 2, 5000, 256, 128, 128, 576
    codes, scales = oracle.quantize(rng.standard_normal((B * N, D)).astype(np.float32))
    kv = api.cache(dev(codes.reshape(B, N, D // 2)), dev(scales.reshape(B, N, D // 16)), D, N)
    q = torch.from_numpy(rng.standard_normal((B, 16, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    idx = dev(np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(B)]).astype(np.int32))
    swa = dev(rng.integers(0, 0x7E, (B, S, D)).astype(np.uint8))
    swa_scale = dev(np.full(B, 0.01, np.float32))
    pos0 = dev(np.full(B, N - S, np.int32))
    q_pos = dev(np.full(B, N - 1, np.int32))
    ws = api.workspace(api.sparse_attn_workspace_bytes(B, K, W, 512))
    out_ref = torch.empty((B, 16, 512), dtype=torch.float32, device="cuda")
    lse_ref = torch.empty((B, 16), dtype=torch.float32, device="cuda")
    api.sparse_attn(q, B, 1, kv, idx, K, swa, swa_scale, pos0, S, W, q_pos, 0.04, 512,
                    out_ref, lse_ref, ws)
    out = torch.zeros_like(out_ref)
    lse = torch.zeros_like(lse_ref)
    api.set_wait_limit(0)
    api.sparse_attn_one_launch(q, B, 1, kv, idx, K, swa, swa_scale, pos0, S, W, q_pos, 0.04, 512,
                               out, lse, ws)
    api.set_wait_limit(1 << 20)
    with pytest.raises(api.Csa2Error) as e:
        api.workspace_check(ws, B)
    assert e.value.status == api.ERR_INCOMPLETE
    api.sparse_attn_one_launch(q, B, 1, kv, idx, K, swa, swa_scale, pos0, S, W, q_pos, 0.04, 512,
                               out, lse, ws)
    api.workspace_check(ws, B)
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
