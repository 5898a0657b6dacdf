"""Pins of the oracle's sparse attention and of the layer modes.

Attention over all positions with no window must equal textbook dense
softmax attention (numpy, over rows decoded independently); with a window it
must equal dense attention over the concatenated rows.  Degenerate cases
(equal keys, one dominant logit, skipped entries) have closed forms.  Modes
(helmcode.com/deepseek-v41-flash, section "03 · CSA2"; 0x0moeen.in/writes/
deepseek-v4-1-flash-kv-cache, "Then every layer stops asking the same
question"): a Reuse layer fed a Full layer's indices, query and window
reproduces it; a Reindex layer fed the Full layer's indexer query reproduces
its selection; a pool at least as large as the context changes nothing; a
one-token prefill chunk equals a decode step.
"""
import numpy as np
import pytest
import torch

from sparse_attention_decode_e2m1_amd import inputs as I
from tests.test_oracle_select import independent_dequant


def dense_attention(q, rows, sm_scale, dv):
    """softmax(q rows^T * s) rows[:, :dv] in float64."""
    logits = (q.astype(np.float64) @ rows.T) * sm_scale
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ rows[:, :dv]) / l, (m + np.log(l))[:, 0]


def fp8_decode(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).double().numpy()


def make_cache(rng, n, d=576):
    x = rng.standard_normal((n, d)).astype(np.float32)
    import oracle
    return oracle.quantize(x)


def test_sparse_equals_dense_no_window(oracle):
    rng = np.random.default_rng(20)
    codes, scales = make_cache(rng, 200)
    q = torch.randn(16, 576).to(torch.bfloat16).float().numpy()
    idx = np.arange(200, dtype=np.int32)
    sm = 1.0 / np.sqrt(576)
    out, lse = oracle.sparse_attn(q, codes, scales, idx, np.zeros((0, 576), np.uint8), 1.0, sm, 512)
    want, wl = dense_attention(q, independent_dequant(codes, scales), sm, 512)
    assert np.allclose(out, want, rtol=1e-11, atol=1e-13)
    assert np.allclose(lse, wl, rtol=1e-12)


def test_sparse_with_window_equals_dense_concat(oracle):
    rng = np.random.default_rng(21)
    codes, scales = make_cache(rng, 300)
    q = torch.randn(16, 576).to(torch.bfloat16).float().numpy()
    idx = np.sort(rng.choice(300, 64, replace=False)).astype(np.int32)
    swa_b, swa_s = I.fp8_rows(torch.randn(128, 576))
    swa = swa_b.numpy()
    sm = 0.05
    out, lse = oracle.sparse_attn(q, codes, scales, idx, swa, swa_s, sm, 512)
    rows = np.concatenate([independent_dequant(codes, scales)[idx], fp8_decode(swa) * swa_s])
    want, wl = dense_attention(q, rows, sm, 512)
    assert np.allclose(out, want, rtol=1e-11, atol=1e-13)
    assert np.allclose(lse, wl, rtol=1e-12)


def test_skipped_entries_and_duplicates(oracle):
    rng = np.random.default_rng(22)
    codes, scales = make_cache(rng, 50)
    q = rng.standard_normal((16, 576)).astype(np.float32)
    idx = np.array([3, -1, 7, -1, 9], np.int32)
    e = np.zeros((0, 576), np.uint8)
    a, la = oracle.sparse_attn(q, codes, scales, idx, e, 1.0, 0.04, 512)
    b, lb = oracle.sparse_attn(q, codes, scales, np.array([3, 7, 9], np.int32), e, 1.0, 0.04, 512)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # the same position twice counts as two entries
    c, lc = oracle.sparse_attn(q, codes, scales, np.array([3, 3], np.int32), e, 1.0, 0.04, 512)
    assert np.allclose(lc, la * 0 + (0.04 * (q.astype(np.float64) @ independent_dequant(codes, scales)[3]) + np.log(2)))


def test_equal_keys_give_mean_of_values(oracle):
    """All logits equal -> output is the plain mean of the value rows."""
    rng = np.random.default_rng(23)
    codes, scales = make_cache(rng, 40)
    q = np.zeros((16, 576), np.float32)
    idx = np.arange(40, dtype=np.int32)
    out, lse = oracle.sparse_attn(q, codes, scales, idx, np.zeros((0, 576), np.uint8), 1.0, 1.0, 512)
    want = independent_dequant(codes, scales)[:, :512].mean(0)
    assert np.allclose(out, want[None, :], rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, np.log(40))


def test_dominant_logit_gives_that_row(oracle):
    rng = np.random.default_rng(24)
    codes, scales = make_cache(rng, 30)
    rows = independent_dequant(codes, scales)
    q = (rows[17] * 100).astype(np.float32)[None, :].repeat(16, 0)
    idx = np.arange(30, dtype=np.int32)
    out, _ = oracle.sparse_attn(q, codes, scales, idx, np.zeros((0, 576), np.uint8), 1.0, 1.0, 512)
    assert np.allclose(out, rows[17, :512][None, :], rtol=0, atol=1e-12)


def test_no_entries(oracle):
    rng = np.random.default_rng(25)
    codes, scales = make_cache(rng, 4)
    out, lse = oracle.sparse_attn(np.ones((16, 576), np.float32), codes, scales,
                                  np.full(8, -1, np.int32), np.zeros((0, 576), np.uint8), 1.0, 1.0, 512)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))


# ----------------------------------------------------------------- modes
def _small():
    return I.small("t_modes", 90, B=1, N=700, K=48, modes=(I.FULL,), W=16)


def _layer(w, b, layer):
    L = I.layer_inputs(w, b, layer)
    return dict(q=L.q.float().numpy(), q_idx=L.q_idx.float().numpy(), w_idx=L.w_idx.numpy(),
                swa=L.swa.numpy(), swa_scale=L.swa_scale, swa_pos0=L.swa_pos0)


def _caches(oracle, w, b):
    c = I.seq_cache(w, b)
    kvc, kvs = oracle.quantize(c.kv.numpy())
    ic, isc = oracle.quantize(c.ikey.numpy())
    return c, kvc, kvs, ic, isc


def test_reuse_reproduces_full_and_reindex_selection(oracle):
    w = _small()
    c, kvc, kvs, ic, isc = _caches(oracle, w, 0)
    L = _layer(w, 0, 0)
    qpos = np.array([w.N - 1])
    full = oracle.layer_step(oracle.FULL, q=L["q"], swa=L["swa"], swa_scale=L["swa_scale"],
                             swa_pos0=L["swa_pos0"], W=w.W, sm_scale=w.sm_scale, dv=w.DV, K=w.K,
                             kv_codes=kvc, kv_scales=kvs, q_pos=qpos, ix_codes=ic, ix_scales=isc,
                             q_idx=L["q_idx"], w_idx=L["w_idx"], new_kv=c.kv.numpy()[qpos],
                             new_ikey=c.ikey.numpy()[qpos], keep_scores=True)
    reuse = oracle.layer_step(oracle.REUSE, q=L["q"], swa=L["swa"], swa_scale=L["swa_scale"],
                              swa_pos0=L["swa_pos0"], W=w.W, sm_scale=w.sm_scale, dv=w.DV, K=w.K,
                              kv_codes=kvc, kv_scales=kvs, q_pos=qpos, idx_in=full.idx)
    assert np.array_equal(reuse.out, full.out) and np.array_equal(reuse.lse, full.lse)
    rein = oracle.layer_step(oracle.REINDEX, q=L["q"], swa=L["swa"], swa_scale=L["swa_scale"],
                             swa_pos0=L["swa_pos0"], W=w.W, sm_scale=w.sm_scale, dv=w.DV, K=w.K,
                             kv_codes=kvc, kv_scales=kvs, q_pos=qpos, ix_codes=ic, ix_scales=isc,
                             q_idx=L["q_idx"], w_idx=L["w_idx"])
    assert np.array_equal(rein.idx, full.idx)
    assert np.array_equal(rein.out, full.out)
    # the selection is the Top-K of the scores by brute force
    from tests.test_oracle_select import brute_topk
    assert list(full.idx[0]) == brute_topk(full.scores[0], w.N, w.K)
    # the FULL write equals a plain quantize of the new row
    nc, ns = oracle.quantize(c.kv.numpy()[qpos])
    assert np.array_equal(kvc[qpos], nc) and np.array_equal(kvs[qpos], ns)


def test_pool_at_least_context_is_flat(oracle):
    w = _small()
    c, kvc, kvs, ic, isc = _caches(oracle, w, 0)
    L = _layer(w, 0, 0)
    qpos = np.array([w.N - 1])
    common = dict(q=L["q"], swa=L["swa"], swa_scale=L["swa_scale"], swa_pos0=L["swa_pos0"], W=w.W,
                  sm_scale=w.sm_scale, dv=w.DV, K=w.K, kv_codes=kvc, kv_scales=kvs, q_pos=qpos,
                  ix_codes=ic, ix_scales=isc, q_idx=L["q_idx"], w_idx=L["w_idx"],
                  new_kv=c.kv.numpy()[qpos], new_ikey=c.ikey.numpy()[qpos])
    flat = oracle.layer_step(oracle.FULL, **common)
    pooled = oracle.layer_step(oracle.FULL, P=1000, **common)
    assert np.array_equal(pooled.idx, flat.idx) and np.array_equal(pooled.out, flat.out)
    assert pooled.pool_count[0] == w.N
    assert list(pooled.pool[0][:w.N]) == list(range(w.N))
    small_pool = oracle.layer_step(oracle.FULL, P=200, **common)
    assert np.array_equal(small_pool.idx, flat.idx)
    assert set(flat.idx[0]) <= set(small_pool.pool[0])
    # a later layer searching that pool with the same indexer query agrees
    rein = oracle.layer_step(oracle.REINDEX, q=L["q"], swa=L["swa"], swa_scale=L["swa_scale"],
                             swa_pos0=L["swa_pos0"], W=w.W, sm_scale=w.sm_scale, dv=w.DV, K=w.K,
                             kv_codes=kvc, kv_scales=kvs, q_pos=qpos, ix_codes=ic, ix_scales=isc,
                             q_idx=L["q_idx"], w_idx=L["w_idx"], pool_in=small_pool.pool,
                             pool_count_in=small_pool.pool_count)
    assert np.array_equal(rein.idx, flat.idx)


def test_prefill_one_token_equals_decode(oracle):
    w = I.small("t_pre", 91, B=1, N=500, K=32, modes=(I.FULL,), W=16, T=1)
    c, kvc, kvs, ic, isc = _caches(oracle, w, 0)
    L = _layer(w, 0, 0)
    qpos = np.array([w.N - 1])
    kw = dict(q=L["q"], swa=L["swa"], swa_scale=L["swa_scale"], swa_pos0=L["swa_pos0"], W=w.W,
              sm_scale=w.sm_scale, dv=w.DV, K=w.K, q_pos=qpos, q_idx=L["q_idx"], w_idx=L["w_idx"],
              new_kv=c.kv.numpy()[qpos], new_ikey=c.ikey.numpy()[qpos])
    a = oracle.layer_step(oracle.FULL, kv_codes=kvc.copy(), kv_scales=kvs.copy(), ix_codes=ic.copy(),
                          ix_scales=isc.copy(), **kw)
    # a 3-token chunk whose last token is the same query sees the same state
    w3 = I.small("t_pre3", 91, B=1, N=500, K=32, modes=(I.FULL,), W=16, T=3)
    q3 = np.concatenate([np.zeros((2, 16, 576), np.float32), L["q"]])
    qi3 = np.concatenate([np.zeros((2, 4, 128), np.float32), L["q_idx"]])
    wi3 = np.concatenate([np.zeros((2, 4), np.float32), L["w_idx"]])
    qpos3 = np.array([w.N - 3, w.N - 2, w.N - 1])
    b = oracle.layer_step(oracle.FULL, q=q3, swa=L["swa"], swa_scale=L["swa_scale"],
                          swa_pos0=L["swa_pos0"], W=w.W, sm_scale=w.sm_scale, dv=w.DV, K=w.K,
                          kv_codes=kvc.copy(), kv_scales=kvs.copy(), ix_codes=ic.copy(),
                          ix_scales=isc.copy(), q_pos=qpos3, q_idx=qi3, w_idx=wi3,
                          new_kv=c.kv.numpy()[qpos3], new_ikey=c.ikey.numpy()[qpos3])
    assert np.array_equal(b.idx[2], a.idx[0])
    assert np.array_equal(b.out[2], a.out[0])
    # causality: the first token of the chunk sees nothing beyond itself
    assert b.idx[0].max() <= w.N - 3


def test_forty_layer_plan_and_window_only_layer(oracle):
    """The 40-layer plan's counts (helmcode.com/deepseek-v41-flash, section
    "03 · CSA2": 4 Full, 4 Reindex, 30 Reuse, 2 window-only) and grouping, and
    a window-only layer equal to dense attention over its window rows."""
    modes = I.forty_layer_modes()
    assert len(modes) == 40 and modes[:2] == (I.SWA, I.SWA)
    assert [modes.count(m) for m in (I.FULL, I.REINDEX, I.REUSE, I.SWA)] == [4, 4, 30, 2]
    g = I.group_of_layers(modes)
    starts = [i for i, m in enumerate(modes) if m == I.FULL]
    assert g[:2] == [0, 0] and [g[i] for i in starts] == [0, 1, 2, 3]
    assert all(modes[i + 1] == I.REINDEX for i in starts)
    from oracle.group import SeqGroup
    w = I.small("t_swa", 91, B=1, N=500, K=32, modes=(I.SWA, I.FULL, I.REUSE), W=16)
    res = SeqGroup(w, 0).step()
    L = I.layer_inputs(w, 0, 0)
    rows = fp8_decode(L.swa.numpy()) * L.swa_scale  # S = W rows, positions N-W .. N-1
    ref_o, ref_l = dense_attention(L.q.float().numpy()[0], rows, w.sm_scale, w.DV)
    assert np.allclose(res[0].out[0], ref_o, rtol=1e-9, atol=1e-12)
    assert np.allclose(res[0].lse[0], ref_l, rtol=1e-9, atol=1e-12)
    assert (res[0].idx.size == 0) or (res[0].idx == -1).all()


# ----------------------------------------------------------------- window rows
def _window_positions_brute(S, pos0, p, W):
    """Every array row (row r holds position pos0 + r) whose position is one
    of the W most recent positions up to and including p."""
    return [pos0 + r for r in range(S) if p - W < pos0 + r <= p]


@pytest.mark.parametrize("W,T,pos0", [(128, 40, 1000), (128, 1, 0), (16, 200, 7), (1, 9, 3)])
def test_window_rows_prefill_chunk_positions(oracle, W, T, pos0):
    """A prefill chunk's window array holds S = W - 1 + T rows (the W - 1
    positions before the chunk, then the chunk's own tokens): token i at
    p = pos0 + W - 1 + i sees exactly positions [p - W + 1, p]."""
    S = W - 1 + T
    tagged = (pos0 + np.arange(S, dtype=np.int64))[:, None]  # each row carries its position
    for i in range(T):
        p = pos0 + W - 1 + i
        got = oracle.window_rows(tagged, pos0, p, W)[:, 0].tolist()
        assert got == _window_positions_brute(S, pos0, p, W) == list(range(p - W + 1, p + 1))
        assert len(got) == W


def test_window_rows_clipped_to_the_array(oracle):
    """Positions outside the array are not invented: a query before the
    array's first W positions sees fewer rows; one past its end sees only
    rows still within its last W positions; W larger than S sees all."""
    S, pos0 = 20, 100
    tagged = (pos0 + np.arange(S, dtype=np.int64))[:, None]
    for W in (1, 5, 20, 64):
        for p in range(pos0 - 3, pos0 + S + 30):
            got = oracle.window_rows(tagged, pos0, p, W)[:, 0].tolist()
            assert got == _window_positions_brute(S, pos0, p, W), (W, p)
    assert oracle.window_rows(tagged, pos0, pos0 - 1, 8).shape[0] == 0
    assert oracle.window_rows(tagged, pos0, pos0 + S + 7, 8).shape[0] == 0


def test_prefill_window_attention_equals_dense_over_brute_window(oracle):
    """A window-only layer over a prefill chunk (S > W): each token's output is
    dense attention over exactly the decoded rows of positions [p - W + 1, p]."""
    from oracle.group import SeqGroup
    w = I.small("t_swa_pre", 92, B=1, N=600, K=32, modes=(I.SWA,), W=16, T=24)
    res = SeqGroup(w, 0).step()[0]
    L = I.layer_inputs(w, 0, 0)
    S = L.swa.shape[0]
    assert S == w.W - 1 + w.T and L.swa_pos0 == w.N - S
    dec = fp8_decode(L.swa.numpy()) * L.swa_scale
    q = L.q.float().numpy()
    for t in range(w.T):
        p = w.ctx0 + t
        pos = _window_positions_brute(S, L.swa_pos0, p, w.W)
        assert len(pos) == w.W and pos[-1] == p
        rows = dec[np.asarray(pos) - L.swa_pos0]
        ref_o, ref_l = dense_attention(q[t], rows, w.sm_scale, w.DV)
        assert np.allclose(res.out[t], ref_o, rtol=1e-9, atol=1e-12), t
        assert np.allclose(res.lse[t], ref_l, rtol=1e-9, atol=1e-12), t
    # an off-by-one (one row too many or too few) changes the result
    p = w.ctx0 + 5
    pos = _window_positions_brute(S, L.swa_pos0, p, w.W + 1)
    wrong, _ = dense_attention(q[5], dec[np.asarray(pos) - L.swa_pos0], w.sm_scale, w.DV)
    assert not np.allclose(res.out[5], wrong, rtol=1e-6, atol=1e-9)
