"""GPU parity of each entry point, called through the C ABI, against the oracle.

Bit-exact: FP4 codes and scale bytes, Top-K index sets fed the same fp32
scores.  Floating point: indexer scores within an fp32-accumulation bound of
the fp64 oracle; attention within max-abs 2e-3 and rel-L2 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_e2m1_amd import api
from sparse_attention_decode_e2m1_amd import inputs as I
from tests.gpu_common import (assert_attention_close, assert_topk_band, dev, host)

pytestmark = pytest.mark.gpu


def setup_module(module):
    print("\n[gpu] device:", torch.cuda.get_device_name(0), flush=True)
    api.lib()


def ctl_words_zero(ws, rows):
    """The per-row control blocks at the start of a workspace are zero."""
    words = ws[: api.lib().csa2_workspace_control_bytes(rows)].view(torch.int32)
    return int(torch.count_nonzero(words)) == 0


# ------------------------------------------------------------ quantize
def special_rows(dim):
    rng = np.random.default_rng(100)
    rows = []
    rows.append(np.zeros(dim))
    rows.append(-np.zeros(dim))
    rows.append(np.full(dim, 1e-30))
    rows.append(rng.standard_normal(dim) * 1e4)          # saturating scales
    rows.append(rng.standard_normal(dim) * 1e-3)         # subnormal scales
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = (e4[:-1] + e4[1:]) / 2
    for j in range(126):                                 # amax exactly 6 x midpoint
        r = rng.standard_normal(dim) * 0.1 * mids[j]
        r[::16] = 6 * mids[j]
        rows.append(r)
    for b in (8, 33, 56, 62, 90, 120):                    # elements exactly on E2M1 midpoints
        s = e4[b]
        t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
        r = np.resize(np.concatenate([t, -t]) * s, dim)
        rows.append(r)
    x = np.stack(rows).astype(np.float32)
    # fp32 neighbours of every value, to probe both sides of each threshold
    up = np.nextafter(x, np.float32(np.inf))
    dn = np.nextafter(x, np.float32(-np.inf))
    return np.concatenate([x, up, dn])


@pytest.mark.parametrize("dim", [576, 128])
def test_quantize_fp32_bit_exact(dim):
    rng = np.random.default_rng(dim)
    x = (rng.standard_normal((3000, dim)) * 10.0 ** rng.uniform(-4, 3, (3000, 1))).astype(np.float32)
    x = np.concatenate([x, special_rows(dim)])
    codes = torch.zeros((x.shape[0], dim // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((x.shape[0], dim // 16), dtype=torch.uint8, device="cuda")
    api.quantize_kv(dev(x), codes, scales)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize(x)
    assert np.array_equal(host(scales), os_)
    assert np.array_equal(host(codes), oc)


def test_quantize_bf16_and_scatter():
    rng = np.random.default_rng(5)
    xb = torch.from_numpy(rng.standard_normal((777, 576)).astype(np.float32)).to(torch.bfloat16)
    dst = torch.from_numpy(rng.permutation(1000)[:777].astype(np.int64))
    codes = torch.zeros((1000, 288), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((1000, 36), dtype=torch.uint8, device="cuda")
    api.quantize_kv(xb.cuda(), codes, scales, dst_rows=dst.cuda())
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize(xb.float().numpy())
    hc, hs = host(codes), host(scales)
    assert np.array_equal(hc[dst.numpy()], oc) and np.array_equal(hs[dst.numpy()], os_)
    untouched = np.setdiff1d(np.arange(1000), dst.numpy())
    assert (hc[untouched] == 0).all()


@pytest.mark.parametrize("dim,rope,dtype", [(576, 64, "f32"), (576, 64, "bf16"), (576, 0, "f32"),
                                             (128, 128, "f32")])
def test_rope_quantize_bit_exact(dim, rope, dtype):
    """Fused rotary step + quantize-on-write against the oracle's rope_quantize
    on the same inputs and angle tables (scattered destination rows)."""
    rng = np.random.default_rng(dim + rope)
    n = 1500
    x = (rng.standard_normal((n, dim)) * 10.0 ** rng.uniform(-3, 2, (n, 1))).astype(np.float32)
    xt = torch.from_numpy(x)
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
        x = xt.float().numpy()
    pos = rng.integers(0, 1 << 20, n)
    cs = I.rope_cos_sin(pos, rope) if rope else torch.zeros((n, 0, 2))
    dst = torch.from_numpy(rng.permutation(2 * n)[:n].astype(np.int64))
    codes = torch.zeros((2 * n, dim // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((2 * n, dim // 16), dtype=torch.uint8, device="cuda")
    api.rope_quantize_kv(xt.cuda(), rope, cs.cuda() if rope else None, codes, scales,
                         dst_rows=dst.cuda())
    torch.cuda.synchronize()
    oc, os_ = oracle.rope_quantize(x, cs.numpy(), rope)
    hc, hs = host(codes), host(scales)
    assert np.array_equal(hs[dst.numpy()], os_)
    assert np.array_equal(hc[dst.numpy()], oc)
    if rope:
        plain_c, _ = oracle.quantize(x)
        assert not np.array_equal(plain_c[:, (dim - rope) // 2:], oc[:, (dim - rope) // 2:])


# ------------------------------------------------------------ index score
def _index_case(seed, B, cap, DI, HI, n_valid):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((B * cap, DI)).astype(np.float32)
    ic, isc = oracle.quantize(keys)
    q = torch.randn(B, HI, DI, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    w = torch.rand(B, HI, generator=torch.Generator().manual_seed(seed + 1))
    return ic, isc, q, w


def _abs_bound(ic, isc, q, w, rows):
    k = oracle.dequant(ic[rows], isc[rows])
    qa = np.abs(q.float().numpy().astype(np.float64))
    return (np.abs(k) @ qa.T * np.abs(w.numpy().astype(np.float64))).sum(1)


@pytest.mark.parametrize("DI,HI", [(128, 4), (128, 1), (128, 16), (256, 4)])
def test_index_score_flat(DI, HI):
    B, cap = 3, 9000
    nv = np.array([9000, 4097, 1], np.int32)
    ic, isc, q, w = _index_case(11 + DI + HI, B, cap, DI, HI, nv)
    scores = torch.full((B, cap), np.nan, device="cuda")
    cache = api.cache(dev(ic), dev(isc), DI, cap)
    api.index_score(cache, B, 1, q.cuda(), w.cuda(), dev(nv), scores)
    torch.cuda.synchronize()
    g = host(scores)
    for b in range(B):
        rows = np.arange(b * cap, b * cap + nv[b])
        o = oracle.index_scores(ic, isc, q[b].float().numpy(), w[b].numpy(), rows)
        bound = _abs_bound(ic, isc, q[b], w[b], rows)
        err = np.abs(g[b, : nv[b]] - o)
        assert (err <= 1e-5 * bound + 1e-30).all(), (b, err.max())
        assert np.isnan(g[b, nv[b]:]).all() or nv[b] == cap  # untouched beyond n_valid


def test_index_score_pool():
    B, cap, P = 2, 20000, 3000
    rng = np.random.default_rng(3)
    ic, isc, q, w = _index_case(21, B, cap, 128, 4, None)
    pool = np.stack([np.sort(rng.choice(cap, P, replace=False)) for _ in range(B)]).astype(np.int32)
    count = np.array([P, 1234], np.int32)
    scores = torch.zeros((B, P), device="cuda")
    cache = api.cache(dev(ic), dev(isc), 128, cap)
    api.index_score(cache, B, 1, q.cuda(), w.cuda(), dev(count), scores, pool=dev(pool))
    torch.cuda.synchronize()
    g = host(scores)
    for b in range(B):
        rows = b * cap + pool[b, : count[b]].astype(np.int64)
        o = oracle.index_scores(ic, isc, q[b].float().numpy(), w[b].numpy(), rows)
        bound = _abs_bound(ic, isc, q[b], w[b], rows)
        assert (np.abs(g[b, : count[b]] - o) <= 1e-5 * bound + 1e-30).all()


def test_index_score_special_cases():
    """One head, w = 1, q = e_c: score = relu(k[c]) exactly; negative query: 0."""
    cap = 3000
    rng = np.random.default_rng(9)
    keys = rng.standard_normal((cap, 128)).astype(np.float32)
    ic, isc = oracle.quantize(keys)
    k_hat = oracle.dequant(ic, isc)
    cache = api.cache(dev(ic), dev(isc), 128, cap)
    for c in (0, 17, 64, 127):
        q = torch.zeros(1, 1, 128)
        q[0, 0, c] = 1.0
        s = torch.zeros((1, cap), device="cuda")
        api.index_score(cache, 1, 1, q.to(torch.bfloat16).cuda(), torch.ones(1, 1).cuda(),
                        dev(np.array([cap], np.int32)), s)
        torch.cuda.synchronize()
        assert np.array_equal(host(s)[0], np.maximum(k_hat[:, c], 0.0).astype(np.float32))
    pos_keys = np.abs(keys)
    pc, ps = oracle.quantize(pos_keys)
    cache2 = api.cache(dev(pc), dev(ps), 128, cap)
    q = -torch.ones(1, 4, 128)
    s = torch.full((1, cap), 5.0, device="cuda")
    api.index_score(cache2, 1, 1, q.to(torch.bfloat16).cuda(), torch.full((1, 4), 0.5).cuda(),
                    dev(np.array([cap], np.int32)), s)
    torch.cuda.synchronize()
    assert (host(s) == 0).all()


# ------------------------------------------------------------ top-k
def _run_topk(scores_np, nv, k, slot_pos=None):
    rows, n = scores_np.shape
    ws = api.workspace(api.topk_workspace_bytes(rows, n, k))
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    api.topk(dev(scores_np), dev(np.asarray(nv, np.int32)), k, idx, ws,
             slot_pos=None if slot_pos is None else dev(slot_pos), count_out=cnt)
    torch.cuda.synchronize()
    assert ctl_words_zero(ws, rows), "control words not cleared"
    return host(idx), host(cnt), ws


def _check_topk(scores_np, nv, k, slot_pos=None):
    g, cnt, _ = _run_topk(scores_np, nv, k, slot_pos)
    for r in range(scores_np.shape[0]):
        sp = None if slot_pos is None else slot_pos[r]
        o, c = oracle.topk(scores_np[r].astype(np.float64), int(nv[r]), k, slot_pos=sp)
        assert np.array_equal(g[r], o), (r, k, int(nv[r]))
        assert cnt[r] == c


@pytest.mark.parametrize("n,k", [(1000, 1), (1000, 7), (4097, 256), (65536 + 5, 2048),
                                 (20000, 16384), (300, 2048)])
def test_topk_random(n, k):
    rng = np.random.default_rng(n + k)
    s = rng.standard_normal((3, n)).astype(np.float32)
    nv = np.array([n, max(1, n // 2 + 3), min(n, k + 1)], np.int32)
    _check_topk(s, nv, k)


def test_topk_ties_and_signed_zero():
    rng = np.random.default_rng(1)
    n = 50000
    s = np.stack([
        np.round(rng.standard_normal(n), 1),          # heavy ties
        np.zeros(n),                                   # one tie storm (overflows the candidates)
        np.where(rng.random(n) < 0.5, -0.0, 0.0),     # -0 == +0
        rng.integers(0, 3, n).astype(np.float64),      # three values
    ]).astype(np.float32)
    nv = np.full(4, n, np.int32)
    for k in (1, 100, 2048, 16384):
        _check_topk(s, nv, k)


def test_topk_large_rows():
    rng = np.random.default_rng(2)
    n = 1 << 20
    s = rng.standard_normal((2, n)).astype(np.float32)
    s[1, 123456] = 50.0
    _check_topk(s, np.array([n, n - 77], np.int32), 2048)
    _check_topk(s[:1], np.array([n], np.int32), 16384)


def test_topk_many_rows():
    # more select blocks than the device holds at once, fewer rows than take
    # one block per row: the path whose last block completes each row
    rng = np.random.default_rng(5)
    rows, n = 48, 100000 + 100
    s = rng.standard_normal((rows, n)).astype(np.float32)
    nv = rng.integers(200, n + 1, rows).astype(np.int32)
    _check_topk(s, nv, 256)


@pytest.mark.parametrize("n", [40007, 12005])
@pytest.mark.parametrize("kind", ["normal", "ties", "three_values", "slot_map"])
def test_topk_one_block_per_row(kind, n):
    """64 or more rows of at most 2^18 slots: one block per row selects in LDS
    (the cut bin's candidates listed there, or, past 4096 of them, further
    passes over the row).  Rows at and below k visible slots included.  Rows
    of 8K to 16K slots keep their keys in registers."""
    rng = np.random.default_rng(len(kind) + n)
    rows = 72
    if kind == "ties":
        s = np.round(rng.standard_normal((rows, n)), 1)
        s[3] = np.where(rng.random(n) < 0.5, -0.0, 0.0)   # -0 == +0
        s[4] = 0.0                                        # one tie storm
    elif kind == "three_values":
        s = rng.integers(0, 3, (rows, n)).astype(np.float64)
    else:
        s = rng.standard_normal((rows, n))
    s = s.astype(np.float32)
    pool = None
    if kind == "slot_map":
        pool = np.stack([np.sort(rng.choice(1 << 20, n, replace=False))
                         for _ in range(rows)]).astype(np.int32)
    for k in (1, 256, 2048):
        nv = rng.integers(k + 1, n + 1, rows).astype(np.int32)
        nv[0], nv[1], nv[2] = max(k - 5, 0), k, k + 1
        _check_topk(s, nv, k, slot_pos=pool)


def test_topk_slot_map():
    rng = np.random.default_rng(4)
    P = 16384
    pool = np.stack([np.sort(rng.choice(1 << 20, P, replace=False)) for _ in range(2)]).astype(np.int32)
    s = rng.standard_normal((2, P)).astype(np.float32)
    _check_topk(s, np.array([P, 9000], np.int32), 2048, slot_pos=pool)


def test_topk_deterministic_and_reusable_workspace():
    rng = np.random.default_rng(6)
    s = np.round(rng.standard_normal((2, 100000)), 2).astype(np.float32)
    nv = np.array([100000, 99999], np.int32)
    g1, _, ws = _run_topk(s, nv, 2048)
    idx = torch.empty((2, 2048), dtype=torch.int32, device="cuda")
    for _ in range(3):  # same workspace, no re-initialisation
        api.topk(dev(s), dev(nv), 2048, idx, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), g1)


# ------------------------------------------------------------ attention
def _attn_case(seed, N, D=576, S=128):
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((N, D)).astype(np.float32)
    codes, scales = oracle.quantize(kv)
    swa_b, swa_s = I.fp8_rows(torch.from_numpy(rng.standard_normal((S, D)).astype(np.float32)))
    return codes, scales, swa_b.numpy(), swa_s


@pytest.mark.parametrize("K,W,npad", [(2048, 128, 0), (2048, 128, 37), (256, 0, 5), (0, 128, 0),
                                      (100, 128, 0), (16, 1, 0)])
def test_sparse_attn_parity(K, W, npad):
    N, T = 6000, 3
    codes, scales, swa, swa_s = _attn_case(K + W, N)
    rng = np.random.default_rng(K * 7 + W)
    idx = np.full((T, max(K, 1)), -1, np.int32)[:, :K]
    for t in range(T):
        sel = np.sort(rng.choice(N, K - npad, replace=False)) if K else np.zeros(0, np.int32)
        idx[t, : len(sel)] = sel
    q = torch.randn(T, 16, 576, generator=torch.Generator().manual_seed(K + W)).to(torch.bfloat16)
    q_pos = np.array([N - 1, N - 50, N - 200], np.int32)   # window partly outside the array
    S = 128
    pos0 = N - S
    sm = 1.0 / np.sqrt(576)
    out = torch.full((T, 16, 512), np.nan, device="cuda")
    lse = torch.full((T, 16), np.nan, device="cuda")
    ws = api.workspace(api.sparse_attn_workspace_bytes(T, K, W, 512))
    kvc = api.cache(dev(codes), dev(scales), 576, N)
    api.sparse_attn(q.cuda(), 1, T, kvc, dev(idx) if K else None, K, dev(swa[None]),
                    dev(np.array([swa_s], np.float32)), dev(np.array([pos0], np.int32)), S, W,
                    dev(q_pos), float(np.float32(sm)), 512, out, lse, ws)
    torch.cuda.synchronize()
    assert ctl_words_zero(ws, T)
    go, gl = host(out), host(lse)
    for t in range(T):
        wrows = oracle.window_rows(swa, pos0, int(q_pos[t]), W)
        o, l = oracle.sparse_attn(q[t].float().numpy(), codes, scales, idx[t], wrows, swa_s,
                                  float(np.float32(sm)), 512)
        assert_attention_close(go[t], o, what=(K, W, t))
        assert np.allclose(gl[t], l, atol=1e-4, rtol=1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_fp8_bit_exact(dtype):
    """FP8 variant of the main cache: bytes and per-row scales equal the
    oracle's (scattered destination rows, rows of very different sizes, an
    all-zero row)."""
    rng = np.random.default_rng(17)
    n = 2000
    x = (rng.standard_normal((n, 576)) * 10.0 ** rng.uniform(-6, 4, (n, 1))).astype(np.float32)
    x[5] = 0.0
    x[9, 100] = 1e30
    xt = torch.from_numpy(x)
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
        x = xt.float().numpy()
    dst = torch.from_numpy(rng.permutation(3 * n)[:n].astype(np.int64))
    codes = torch.zeros((3 * n, 576), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((3 * n,), dtype=torch.float32, device="cuda")
    api.quantize_kv_fp8(xt.cuda(), codes, scales, dst_rows=dst.cuda())
    torch.cuda.synchronize()
    ob, os_ = oracle.quantize_fp8(x)
    d = dst.numpy()
    assert np.array_equal(host(scales)[d].view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(host(codes)[d], ob)


@pytest.mark.parametrize("K,W,npad", [(2048, 128, 0), (2048, 128, 37), (256, 0, 5), (100, 128, 0)])
def test_sparse_attn_fp8_parity(K, W, npad):
    """Attention over an FP8 main cache against the oracle's float64
    definition, at the FP4 attention's tolerance."""
    N, T = 6000, 3
    rng = np.random.default_rng(K + 3 * W + npad)
    kv = (rng.standard_normal((N, 576)) * rng.uniform(0.5, 1.5, (N, 1))).astype(np.float32)
    b8, s8 = oracle.quantize_fp8(kv)
    swa_b, swa_s = I.fp8_rows(torch.from_numpy(rng.standard_normal((128, 576)).astype(np.float32)))
    swa = swa_b.numpy()
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        sel = np.sort(rng.choice(N, K - npad, replace=False))
        idx[t, : len(sel)] = sel
    q = torch.randn(T, 16, 576, generator=torch.Generator().manual_seed(K + W + 1)).to(torch.bfloat16)
    q_pos = np.array([N - 1, N - 50, N - 200], np.int32)
    S, pos0 = 128, N - 128
    sm = float(np.float32(1.0 / np.sqrt(576)))
    out = torch.full((T, 16, 512), np.nan, device="cuda")
    lse = torch.full((T, 16), np.nan, device="cuda")
    ws = api.workspace(api.sparse_attn_workspace_bytes(T, K, W, 512))
    kv8 = api.fp8_cache(dev(b8), dev(s8), 576, N)
    api.sparse_attn_fp8(q.cuda(), 1, T, kv8, dev(idx), K, dev(swa[None]),
                        dev(np.array([swa_s], np.float32)), dev(np.array([pos0], np.int32)), S, W,
                        dev(q_pos), sm, 512, out, lse, ws)
    torch.cuda.synchronize()
    assert ctl_words_zero(ws, T)
    go, gl = host(out), host(lse)
    for t in range(T):
        wrows = oracle.window_rows(swa, pos0, int(q_pos[t]), W)
        o, l = oracle.sparse_attn_fp8(q[t].float().numpy(), b8, s8, idx[t], wrows, swa_s, sm, 512)
        assert_attention_close(go[t], o, what=(K, W, t))
        assert np.allclose(gl[t], l, atol=1e-4, rtol=1e-5)


def test_sparse_attn_no_entries():
    N = 100
    codes, scales, swa, swa_s = _attn_case(1, N)
    q = torch.randn(1, 16, 576).to(torch.bfloat16)
    idx = np.full((1, 64), -1, np.int32)
    out = torch.full((1, 16, 512), np.nan, device="cuda")
    lse = torch.zeros((1, 16), device="cuda")
    ws = api.workspace(api.sparse_attn_workspace_bytes(1, 64, 0, 512))
    api.sparse_attn(q.cuda(), 1, 1, api.cache(dev(codes), dev(scales), 576, N), dev(idx), 64,
                    None, None, None, 0, 0, dev(np.array([N - 1], np.int32)), 0.04, 512, out, lse, ws)
    torch.cuda.synchronize()
    assert (host(out) == 0).all() and np.isneginf(host(lse)).all()


def test_sparse_attn_window_without_rows():
    """W > 0 over an empty window array (S = 0, no window pointers): only the
    Top-K entries are attended."""
    N, K = 3000, 200
    codes, scales, _, _ = _attn_case(5, N)
    rng = np.random.default_rng(5)
    idx = np.sort(rng.choice(N, K, replace=False)).astype(np.int32)[None]
    q = torch.randn(1, 16, 576, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    out = torch.full((1, 16, 512), np.nan, device="cuda")
    lse = torch.full((1, 16), np.nan, device="cuda")
    ws = api.workspace(api.sparse_attn_workspace_bytes(1, K, 128, 512))
    sm = float(np.float32(0.05))
    api.sparse_attn(q.cuda(), 1, 1, api.cache(dev(codes), dev(scales), 576, N), dev(idx), K,
                    None, None, None, 0, 128, dev(np.array([N - 1], np.int32)), sm, 512, out, lse, ws)
    torch.cuda.synchronize()
    o, l = oracle.sparse_attn(q[0].float().numpy(), codes, scales, idx[0],
                              np.zeros((0, 576), np.uint8), 1.0, sm, 512)
    assert_attention_close(host(out)[0], o, what="S=0")
    assert np.allclose(host(lse)[0], l, atol=1e-4, rtol=1e-5)


def _attn_batch(B, T, N, K, npad, D, seed):
    """Seeded attention inputs: B sequences of T decode rows over an FP4 cache
    of N rows each, a window per sequence, K sorted Top-K entries per row (the
    last npad of them -1)."""
    rng = np.random.default_rng(seed)
    codes, scales = oracle.quantize(rng.standard_normal((B * N, D)).astype(np.float32))
    S = 128 if D == 576 else 64
    sw = [I.fp8_rows(torch.from_numpy(rng.standard_normal((S, D)).astype(np.float32)))
          for _ in range(B)]
    swa = np.stack([s[0].numpy() for s in sw])
    swa_s = np.array([s[1] for s in sw], np.float32)
    rows = B * T
    idx = np.full((rows, K), -1, np.int32)
    for r in range(rows):
        sel = np.sort(rng.choice(N, K - npad, replace=False))
        idx[r, : len(sel)] = sel
    q = torch.from_numpy(rng.standard_normal((rows, 16, D)).astype(np.float32)).to(torch.bfloat16)
    q_pos = np.array([N - 1 - 7 * (r % T) for r in range(rows)], np.int32)
    pos0 = np.full(B, N - S, np.int32)
    return codes, scales, swa, swa_s, idx, q, q_pos, pos0, S


@pytest.mark.parametrize("B,T,N,K,W,npad,D", [
    (4, 1, 6000, 2048, 128, 0, 576),   # the decode group's grid: 4 rows x 34 splits
    (1, 3, 6000, 2048, 128, 37, 576),
    (2, 2, 3000, 100, 128, 0, 576),
    (2, 1, 3000, 256, 0, 5, 576),      # no window
    (3, 1, 2000, 300, 64, 0, 128),     # the 128-channel kernel
    (16, 4, 3000, 2048, 128, 0, 576),  # 64 rows x 34 splits: more blocks than the device holds
])
def test_sparse_attn_one_launch(B, T, N, K, W, npad, D):
    """csa2_sparse_attn_one_launch equals csa2_sparse_attn bit for bit (the
    same split arithmetic and merge grouping; the split + merge kernels when
    the grid does not fit the device at once), matches the oracle, and leaves
    the control words zero for the next call on the same workspace."""
    codes, scales, swa, swa_s, idx, q, q_pos, pos0, S = _attn_batch(B, T, N, K, npad, D, K + B)
    dv = 512 if D == 576 else 128
    rows = B * T
    sm = float(np.float32(1.0 / np.sqrt(D)))
    args = (q.cuda(), B, T, api.cache(dev(codes), dev(scales), D, N), dev(idx), K, dev(swa),
            dev(swa_s), dev(pos0), S, W, dev(q_pos), sm, dv)
    ws = api.workspace(api.sparse_attn_workspace_bytes(rows, K, W, dv))
    ref_o = torch.full((rows, 16, dv), np.nan, device="cuda")
    ref_l = torch.full((rows, 16), np.nan, device="cuda")
    api.sparse_attn(*args, ref_o, ref_l, ws)
    for _ in range(2):
        out = torch.full((rows, 16, dv), np.nan, device="cuda")
        lse = torch.full((rows, 16), np.nan, device="cuda")
        api.sparse_attn_one_launch(*args, out, lse, ws)
        torch.cuda.synchronize()
        assert ctl_words_zero(ws, rows)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    go, gl = host(out), host(lse)
    for r in (0, rows - 1):
        b = r // T
        wrows = oracle.window_rows(swa[b], int(pos0[b]), int(q_pos[r]), W)
        o, l = oracle.sparse_attn(q[r].float().numpy(), codes[b * N:(b + 1) * N],
                                  scales[b * N:(b + 1) * N], idx[r], wrows, float(swa_s[b]), sm, dv)
        assert_attention_close(go[r], o, what=(B, T, K, r))
        assert np.allclose(gl[r], l, atol=1e-4, rtol=1e-5)


@pytest.mark.parametrize("B,T,N,K,W,npad,D", [
    (32, 4, 3000, 2048, 128, 0, 576),    # 128 rows: splits of 4 rounds
    (32, 4, 3000, 2048, 0, 300, 576),    # no window, every row padded
    (64, 4, 3000, 2048, 64, 0, 128),     # the 128-channel kernel, 8 rounds
])
def test_sparse_attn_multi_round(B, T, N, K, W, npad, D):
    """Grids of more than four times the blocks the device holds run splits
    of several rounds (each prefetching the next round's rows): every row
    matches the oracle, a second call on the same workspace gives the same
    bits, and the control words are left zero."""
    codes, scales, swa, swa_s, idx, q, q_pos, pos0, S = _attn_batch(B, T, N, K, npad, D,
                                                                    K + B + W + npad)
    dv = 512 if D == 576 else 128
    rows = B * T
    sm = float(np.float32(1.0 / np.sqrt(D)))
    args = (q.cuda(), B, T, api.cache(dev(codes), dev(scales), D, N), dev(idx), K, dev(swa),
            dev(swa_s), dev(pos0), S, W, dev(q_pos), sm, dv)
    ws = api.workspace(api.sparse_attn_workspace_bytes(rows, K, W, dv))
    res = []
    for _ in range(2):
        out = torch.full((rows, 16, dv), np.nan, device="cuda")
        lse = torch.full((rows, 16), np.nan, device="cuda")
        api.sparse_attn(*args, out, lse, ws)
        torch.cuda.synchronize()
        assert ctl_words_zero(ws, rows)
        res.append((out, lse))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    go, gl = host(res[0][0]), host(res[0][1])
    for r in range(rows):
        b = r // T
        wrows = oracle.window_rows(swa[b], int(pos0[b]), int(q_pos[r]), W)
        o, l = oracle.sparse_attn(q[r].float().numpy(), codes[b * N:(b + 1) * N],
                                  scales[b * N:(b + 1) * N], idx[r], wrows, float(swa_s[b]), sm, dv)
        assert_attention_close(go[r], o, what=(B, T, K, W, r))
        assert np.allclose(gl[r], l, atol=1e-4, rtol=1e-5)


def test_sparse_attn_small_dims_and_batch():
    """D = dv = 128 kernel variant, several sequences."""
    B, N, K = 3, 2000, 300
    rng = np.random.default_rng(8)
    kv = rng.standard_normal((B * N, 128)).astype(np.float32)
    codes, scales = oracle.quantize(kv)
    swa_list = [I.fp8_rows(torch.from_numpy(rng.standard_normal((64, 128)).astype(np.float32)))
                for _ in range(B)]
    swa = np.stack([s[0].numpy() for s in swa_list])
    swa_s = np.array([s[1] for s in swa_list], np.float32)
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(B)]).astype(np.int32)
    q = torch.randn(B, 16, 128).to(torch.bfloat16)
    q_pos = np.full(B, N - 1, np.int32)
    pos0 = np.full(B, N - 64, np.int32)
    out = torch.zeros((B, 16, 128), device="cuda")
    ws = api.workspace(api.sparse_attn_workspace_bytes(B, K, 64, 128))
    api.sparse_attn(q.cuda(), B, 1, api.cache(dev(codes), dev(scales), 128, N), dev(idx), K,
                    dev(swa), dev(swa_s), dev(pos0), 64, 64, dev(q_pos), 0.09, 128, out, None, ws)
    torch.cuda.synchronize()
    for b in range(B):
        o, _ = oracle.sparse_attn(q[b].float().numpy(), codes[b * N:(b + 1) * N],
                                  scales[b * N:(b + 1) * N], idx[b], swa[b], float(swa_s[b]),
                                  float(np.float32(0.09)), 128)
        assert_attention_close(host(out)[b], o, what=b)
