"""Pins of the oracle's indexer score and Top-K selection.

Top-K is checked against Python's own sort of (-score, slot) pairs on tiny
inputs with tie storms; the indexer score is checked against special cases
that reduce to a single dequantized channel, against an independent numpy
evaluation over a cache decoded with the literal E2M1 table and torch's E4M3
decoder, and against its algebraic invariants.  Selection of 512 global
entries from the indexer scores is described on
louisbouchard.ai/deepseek-v41-flash-kv-cache-writing-benchmark ("Share the
cache and the search work").
"""
import numpy as np
import pytest
import torch

from tests.test_oracle_codec import golden_e2m1, torch_e4m3


def brute_topk(scores, n_valid, k, slot_pos=None):
    order = sorted(range(n_valid), key=lambda i: (-float(scores[i]), i))
    take = order[:k]
    pos = [int(slot_pos[i]) if slot_pos is not None else i for i in take]
    pos.sort()
    return pos + [-1] * (k - len(pos))


@pytest.mark.parametrize("seed", range(12))
def test_topk_bruteforce_with_ties(oracle, seed):
    rng = np.random.default_rng(seed)
    for n in (1, 2, 7, 31, 64):
        # few distinct values: tie storms at the k-th score
        scores = rng.integers(-3, 4, n).astype(np.float64)
        scores[rng.random(n) < 0.2] = -0.0
        for k in sorted({1, max(1, n - 1), n, n + 5}):
            for n_valid in sorted({n, max(0, n - 3)}):
                got, cnt = oracle.topk(scores, n_valid, k)
                want = brute_topk(scores, n_valid, k)
                assert list(got) == want, (n, k, n_valid)
                assert cnt == min(k, n_valid)


def test_topk_signed_zero_equal(oracle):
    s = np.array([-0.0, 0.0, -0.0, 0.0, -1.0])
    got, _ = oracle.topk(s, 5, 2)
    assert list(got) == [0, 1]
    got, _ = oracle.topk(s[::-1].copy(), 5, 2)
    assert list(got) == [1, 2]


def test_topk_all_equal(oracle):
    s = np.zeros(50)
    got, _ = oracle.topk(s, 50, 7)
    assert list(got) == list(range(7))


def test_topk_slot_map(oracle):
    rng = np.random.default_rng(5)
    pool = np.sort(rng.choice(1000, 40, replace=False)).astype(np.int32)
    s = rng.standard_normal(40)
    got, _ = oracle.topk(s, 40, 9, slot_pos=pool)
    assert list(got) == brute_topk(s, 40, 9, pool)


def test_topk_pool_then_k_equals_flat(oracle):
    """Selecting K inside the top-P pool gives the flat Top-K (K <= P)."""
    rng = np.random.default_rng(6)
    s = np.round(rng.standard_normal(3000), 1)  # many ties
    flat, _ = oracle.topk(s, 3000, 50)
    pool, cnt = oracle.topk(s, 3000, 400)
    inner, _ = oracle.topk(s[pool[:cnt]], cnt, 50, slot_pos=pool)
    assert list(inner) == list(flat)
    assert set(flat) <= set(pool)


def independent_dequant(codes, scales):
    g = np.array([golden_e2m1()[c] for c in range(16)])
    e4 = torch_e4m3()
    lo = g[codes & 15]
    hi = g[codes >> 4]
    vals = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    sc = np.repeat(e4[scales], 16, axis=1)
    return vals * sc


def test_dequant_matches_independent_decode(oracle):
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, (64, 64), dtype=np.uint8)
    scales = rng.integers(0, 127, (64, 8), dtype=np.uint8)
    assert np.array_equal(oracle.dequant(codes, scales), independent_dequant(codes, scales))


def test_index_score_single_channel(oracle):
    """One head, w = 1, q = unit vector e_c: score = relu(k_hat[c])."""
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((100, 128)).astype(np.float32)
    codes, scales = oracle.quantize(keys)
    k_hat = independent_dequant(codes, scales)
    rows = np.arange(100)
    for c in (0, 1, 15, 16, 63, 127):
        q = np.zeros((1, 128), np.float32)
        q[0, c] = 1.0
        s = oracle.index_scores(codes, scales, q, np.ones(1, np.float32), rows)
        assert np.array_equal(s, np.maximum(k_hat[:, c], 0.0))


def test_index_score_negative_query_gives_zero(oracle):
    keys = np.abs(np.random.default_rng(9).standard_normal((50, 128))).astype(np.float32)
    codes, scales = oracle.quantize(keys)
    q = -np.ones((4, 128), np.float32)
    s = oracle.index_scores(codes, scales, q, np.full(4, 0.5, np.float32), np.arange(50))
    assert np.all(s == 0.0)


def test_index_score_matches_numpy(oracle):
    rng = np.random.default_rng(10)
    keys = rng.standard_normal((300, 128)).astype(np.float32)
    codes, scales = oracle.quantize(keys)
    q = torch.randn(4, 128).to(torch.bfloat16).float().numpy()
    w = rng.random(4).astype(np.float32)
    rows = rng.choice(300, 120, replace=False)
    s = oracle.index_scores(codes, scales, q, w, rows)
    k_hat = independent_dequant(codes, scales)[rows]
    want = (np.maximum(k_hat @ q.astype(np.float64).T, 0.0) * w.astype(np.float64)).sum(1)
    assert np.allclose(s, want, rtol=1e-12, atol=1e-12)


def test_index_score_invariants(oracle):
    """Positively homogeneous in w, additive over heads, invariant to the
    order in which rows are listed."""
    rng = np.random.default_rng(11)
    keys = rng.standard_normal((80, 128)).astype(np.float32)
    codes, scales = oracle.quantize(keys)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    w = rng.random(4).astype(np.float32)
    rows = np.arange(80)
    s = oracle.index_scores(codes, scales, q, w, rows)
    s2 = oracle.index_scores(codes, scales, q, (2 * w).astype(np.float32), rows)
    assert np.allclose(s2, 2 * s, rtol=1e-14)
    parts = sum(oracle.index_scores(codes, scales, q[h:h + 1], w[h:h + 1], rows) for h in range(4))
    assert np.allclose(parts, s, rtol=1e-13)
    perm = rng.permutation(80)
    assert np.array_equal(oracle.index_scores(codes, scales, q, w, perm), s[perm])
