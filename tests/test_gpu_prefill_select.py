"""GPU tests of the prefill selection without a score matrix
(CSA2_TOPK_SAMPLED): on the same inputs it must give the same index rows,
in the same order, as the score-matrix path (CSA2_TOPK_ROW), whether the
rows finish from their candidates or go to the exact path (forced for every
row, or reached by rows whose kept positions overflow), and its selection
must match the oracle's."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_e2m1_amd import api
from sparse_attention_decode_e2m1_amd import harness as Hn
from sparse_attention_decode_e2m1_amd import inputs as I
from tests.gpu_common import compare_group, expected_rows, host
from tests.oracle_runner import run_group

pytestmark = pytest.mark.gpu


def _idx_with(dw, variant):
    """idx_out of the Full layer run with a forced Top-K variant, and the
    variant the pass reported."""
    prev = api.set_topk_variant(variant)
    try:
        dw.layers[0].idx_out.fill_(-7)
        dw.run_layer(0)
        torch.cuda.synchronize()
        return host(dw.layers[0].idx_out).copy(), api.topk_last_variant()
    finally:
        api.set_topk_variant(prev)


def _three_ways(dw):
    a, va = _idx_with(dw, api.TOPK_AUTO)
    r, vr = _idx_with(dw, api.TOPK_ROW)
    f, vf = _idx_with(dw, api.TOPK_SAMPLED_FALLBACK)
    assert va == api.TOPK_SAMPLED and vf == api.TOPK_SAMPLED_FALLBACK and vr == api.TOPK_ROW
    assert (a != -7).all()
    assert np.array_equal(a, r), int((a != r).any(axis=1).sum())
    assert np.array_equal(f, r)
    return a


@pytest.mark.parametrize("K,hi", [(256, 4), (2048, 4), (256, 2), (256, 1), (1, 4), (33, 4)])
def test_sampled_prefill_equals_score_matrix_path(K, hi):
    w = I.small("t_samp", 70 + K % 7 + hi, B=1, N=40000, T=64, K=K, modes=(I.FULL,), HI=hi)
    dw = Hn.DeviceWorkload(w)
    a = _three_ways(dw)
    # every row keeps K distinct visible positions, in ascending order
    for row in a:
        assert (np.diff(row) > 0).all() and row[0] >= 0 and row[-1] < w.N


def test_sampled_prefill_matches_oracle():
    w = I.small("t_samp_o", 71, B=2, N=36000, T=32, K=1024, modes=(I.FULL,))
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    assert api.topk_last_variant() == api.TOPK_SAMPLED
    ores, oc = run_group(w, keep_scores=True)
    chk = compare_group(w, dw, ores, oc)
    assert chk.rows == expected_rows(w) and chk.same_sets >= 32


def test_sampled_prefill_short_rows():
    """Tokens that see fewer positions than K take every visible position
    (the rest -1); tokens just above K select among few samples."""
    w = I.small("t_samp_s", 72, B=1, N=40000, T=64, K=512, modes=(I.FULL,))
    dw = Hn.DeviceWorkload(w)
    # tokens at positions 300..(300+63) of the cache see 301..364 positions;
    # then a second run with tokens around K
    for p0 in (300, 520, 9000):
        dw.q_pos.copy_(torch.arange(p0, p0 + w.T, dtype=torch.int32))
        a = _three_ways(dw)
        for t, row in enumerate(a):
            nv = p0 + t + 1
            if nv <= w.K:
                assert list(row[:nv]) == list(range(nv)) and (row[nv:] == -1).all()


def test_sampled_prefill_ties_overflow_to_exact_path():
    """A sequence whose cached index keys are all zero scores every cached
    position equally: its rows hold far more candidates than there is room
    for and take the exact path, while the other sequence's rows finish from
    their candidates; every row equals the score-matrix path's."""
    w = I.small("t_samp_t", 73, B=2, N=40000, T=32, K=512, modes=(I.FULL,))
    dw = Hn.DeviceWorkload(w)
    kvc, kvs, ixc, ixs = dw.caches[0]
    ixc[1].zero_()
    ixs[1].zero_()
    a = _three_ways(dw)
    # the tied rows keep the new (nonzero) positions first, then the lowest
    # tied slots
    tied = a[w.T:]
    assert (tied[:, 0] == 0).all()


def test_sampled_prefill_multi_pass_against_oracle():
    """2560 query tokens: one pass of 2048 rows and one of 512, each attending
    in launches of at most 1024 rows (1024 + 1024, then 512); tokens at every
    pass and launch boundary match the oracle."""
    w = I.small("t_samp_mp", 74, B=1, N=40000, T=2560, K=256, modes=(I.FULL,))
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    assert api.topk_last_variant() == api.TOPK_SAMPLED
    rng = np.random.default_rng(74)
    fixed = {0, 1, 1023, 1024, 2047, 2048, 2049, w.T - 2, w.T - 1}
    rest = [t for t in rng.permutation(w.T).tolist() if t not in fixed][: 16 - len(fixed)]
    tok = sorted(fixed | set(rest))
    ores, oc = run_group(w, tokens=tok, keep_scores=True)
    chk = compare_group(w, dw, ores, oc, tokens=tok)
    assert chk.rows == expected_rows(w, tokens=tok) and chk.same_sets >= len(tok) // 2

