"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
and the comparison rules (bit-exact bytes and indices; Top-K sets equal or
differing only among scores within 1e-6 relative of the K-th score;
attention within max-abs 2e-3 and rel-L2 1e-3 of the fp64 oracle).

Where the GPU's selection differs from the oracle's inside the tie band, the
attention that follows is still compared: the oracle attends over the GPU's
own indices (and a Reindex layer searching the GPU's pool is re-selected by
the oracle inside that pool), so every row of every layer is checked."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle
from sparse_attention_decode_e2m1_amd import inputs as I

TOPK_BAND = 1e-6
ATT_MAX_ABS = 2e-3
ATT_REL_L2 = 1e-3


def dev(x, dtype=None):
    t = torch.as_tensor(x)
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_topk_band(gpu_idx, ora_idx, ora_scores, k, slot_pos=None, what=""):
    """GPU and oracle Top-K sets may differ only among entries whose oracle
    score lies within TOPK_BAND (relative) of the oracle's k-th score.
    Returns the size of the symmetric difference."""
    g = set(int(x) for x in gpu_idx if x >= 0)
    o = set(int(x) for x in ora_idx if x >= 0)
    assert len(g) == len(o), (what, len(g), len(o))
    assert list(gpu_idx) == sorted(gpu_idx[gpu_idx >= 0].tolist()) + [-1] * int((gpu_idx < 0).sum())
    if g == o:
        return 0
    # scores by position
    if slot_pos is not None:
        pos_score = {int(p): float(s) for p, s in zip(slot_pos, ora_scores)}
    else:
        pos_score = {i: float(s) for i, s in enumerate(ora_scores)}
    kth = min(pos_score[p] for p in o)
    tol = TOPK_BAND * max(abs(kth), 1e-300)
    for p in g ^ o:
        assert p in pos_score, (what, "selected a slot outside the scored list", p)
        assert abs(pos_score[p] - kth) <= tol, (what, p, pos_score[p], kth)
    return len(g ^ o)


def assert_attention_close(gpu_out, ora_out, what=""):
    g = np.asarray(gpu_out, np.float64)
    o = np.asarray(ora_out, np.float64)
    err = np.abs(g - o)
    assert np.isfinite(g).all(), what
    assert err.max() <= ATT_MAX_ABS, (what, err.max())
    rel = np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-30)
    assert rel <= ATT_REL_L2, (what, rel)
    return err.max(), rel


@dataclass
class GroupCheck:
    rows: int = 0            # (sequence, layer, token) rows whose attention was compared
    same_sets: int = 0       # Full/Reindex rows whose Top-K set equals the oracle's exactly
    band_sets: int = 0       # ... that differ inside the tie band (attention then on GPU indices)
    pools: int = 0           # pools compared (Full layers with P > 0)
    reselected: int = 0      # Reindex rows re-selected by the oracle inside the GPU's pool


def _oracle_attention(w, b, li, t, idx, ocache):
    """The oracle's attention for token t of sequence b at layer li over the
    given Top-K indices (the GPU's own selection)."""
    L = I.layer_inputs(w, b, li)
    p = w.ctx0 + t
    wrows = oracle.window_rows(L.swa.numpy(), L.swa_pos0, p, w.W)
    return oracle.sparse_attn(L.q[t].float().numpy(), ocache[0], ocache[1], np.asarray(idx, np.int32),
                              wrows, L.swa_scale, w.sm_scale, w.DV)


def compare_group(w, dw, ores, ocaches, seqs=None, tokens=None) -> GroupCheck:
    """Compare every layer of the device run with the oracle's, row by row:
    caches bit-exact, pools and Top-K sets under the tie rule, and the
    attention of every (sequence, layer, token) row."""
    seqs = list(range(w.B)) if seqs is None else seqs
    tok = list(range(w.T)) if tokens is None else tokens
    kvc, kvs, ixc, ixs = (host(t) for t in dw.caches[0])
    for extra in dw.caches[1:]:  # every group's copy holds the same rows after the step
        for a, t in zip((kvc, kvs, ixc, ixs), extra):
            assert np.array_equal(a, host(t))
    chk = GroupCheck()
    host_idx = [host(L.idx_out) if L.mode in (I.FULL, I.REINDEX) else None for L in dw.layers]
    for b in seqs:
        okvc, okvs, oixc, oixs = ocaches[b]
        assert np.array_equal(kvc[b], okvc) and np.array_equal(kvs[b], okvs), b
        assert np.array_equal(ixc[b], oixc) and np.array_equal(ixs[b], oixs), b
        for li, L in enumerate(dw.layers):
            r = ores[b][li]
            gout = host(L.out)
            glse = host(L.lse)
            for j, t in enumerate(tok):
                row = b * w.T + t
                what = (w.name, b, li, t)
                ora_out, ora_lse = r.out[j], r.lse[j]
                if L.mode in (I.FULL, I.REINDEX):
                    gidx = host_idx[li][row]
                    sp, ref_idx, ref_scores = None, r.idx[j], r.scores[j]
                    if L.mode == I.FULL and w.P > 0:
                        g_pool = host(L.pool_out)[row]
                        assert host(L.pool_count)[row] == r.pool_count[j], what
                        assert_topk_band(g_pool, r.pool[j], r.scores[j], w.P, what=what + ("pool",))
                        chk.pools += 1
                    if L.mode == I.REINDEX and w.P > 0:
                        full = next(x for x in range(li) if dw.layers[x].mode == I.FULL)
                        g_pool = host(dw.layers[full].pool_out)[row]
                        cnt = int(host(dw.layers[full].pool_count)[row])
                        o_pool = ores[b][full].pool[j]
                        if np.array_equal(g_pool, o_pool):
                            sp = o_pool[: ores[b][full].pool_count[j]]
                        else:
                            # the GPU's pool differs inside the band: the oracle
                            # selects inside that pool, as the GPU layer did
                            Li = I.layer_inputs(w, b, li)
                            sp = g_pool[:cnt]
                            ref_scores = oracle.index_scores(
                                ocaches[b][2], ocaches[b][3], Li.q_idx[t].float().numpy(),
                                Li.w_idx[t].numpy(), sp.astype(np.int64))
                            ref_idx, _ = oracle.topk(ref_scores, cnt, w.K, slot_pos=g_pool)
                            chk.reselected += 1
                    nd = assert_topk_band(gidx, ref_idx, ref_scores, w.K, slot_pos=sp, what=what)
                    if nd == 0 and np.array_equal(ref_idx, r.idx[j]):
                        chk.same_sets += 1
                    else:
                        chk.band_sets += int(nd > 0)
                        ora_out, ora_lse = _oracle_attention(w, b, li, t, gidx, ocaches[b])
                elif L.mode == I.REUSE:
                    src = [x for x in range(li) if dw.layers[x].mode in (I.FULL, I.REINDEX)]
                    if src:
                        gsrc = host_idx[src[-1]][row]
                        if not np.array_equal(gsrc, ores[b][src[-1]].idx[j]):
                            ora_out, ora_lse = _oracle_attention(w, b, li, t, gsrc, ocaches[b])
                assert_attention_close(gout[row], ora_out, what=what)
                assert np.allclose(glse[row], ora_lse, atol=1e-4, rtol=1e-5), what
                chk.rows += 1
    return chk


def expected_rows(w, seqs=None, tokens=None) -> int:
    """Rows compare_group must have compared: every (sequence, layer, token)."""
    nb = w.B if seqs is None else len(seqs)
    nt = w.T if tokens is None else len(tokens)
    return nb * len(w.modes) * nt
