"""Runs the oracle over a synthetic workload's layer group (test
infrastructure): the same seeded inputs as the device harness, its own FP4
caches (oracle.quantize), the same static wiring of modes."""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

import oracle
from sparse_attention_decode_e2m1_amd import inputs as I


def run_group(w: I.Workload, seqs: Optional[List[int]] = None,
              tokens: Optional[List[int]] = None, keep_scores: bool = False):
    """Returns {b: [LayerResult per layer]} and the oracle caches per b.
    ``tokens`` (indices into the T query tokens) samples a prefill chunk; the
    Full layer still writes all T rows first."""
    seqs = list(range(w.B)) if seqs is None else seqs
    tok = list(range(w.T)) if tokens is None else tokens
    results: Dict[int, list] = {}
    caches = {}
    for b in seqs:
        c = I.seq_cache(w, b)
        kv = c.kv.numpy()
        ik = c.ikey.numpy()
        kvc, kvs = oracle.quantize(kv[: w.ctx0])
        ixc, ixs = oracle.quantize(ik[: w.ctx0])
        kvc = np.concatenate([kvc, np.zeros((w.T, w.D // 2), np.uint8)])
        kvs = np.concatenate([kvs, np.zeros((w.T, w.D // 16), np.uint8)])
        ixc = np.concatenate([ixc, np.zeros((w.T, w.DI // 2), np.uint8)])
        ixs = np.concatenate([ixs, np.zeros((w.T, w.DI // 16), np.uint8)])
        all_pos = np.arange(w.ctx0, w.N)
        q_pos = all_pos[tok]
        res = []
        last_idx = None
        pool = None
        for li, mode in enumerate(w.modes):
            L = I.layer_inputs(w, b, li)
            q = L.q.float().numpy()[tok]
            qi = L.q_idx.float().numpy()[tok]
            wi = L.w_idx.numpy()[tok]
            common = dict(q=q, swa=L.swa.numpy(), swa_scale=L.swa_scale, swa_pos0=L.swa_pos0,
                          W=w.W, sm_scale=w.sm_scale, dv=w.DV, K=w.K, kv_codes=kvc,
                          kv_scales=kvs, q_pos=q_pos, keep_scores=keep_scores)
            if mode == I.FULL:
                r = oracle.layer_step(oracle.FULL, ix_codes=ixc, ix_scales=ixs, q_idx=qi,
                                      w_idx=wi, new_kv=kv[w.ctx0:], new_ikey=ik[w.ctx0:],
                                      write_pos=all_pos, P=w.P, **common)
                if w.P > 0:
                    pool = (r.pool, r.pool_count)
            elif mode == I.REINDEX:
                kw = {}
                if pool is not None:
                    kw = dict(pool_in=pool[0], pool_count_in=pool[1])
                r = oracle.layer_step(oracle.REINDEX, ix_codes=ixc, ix_scales=ixs, q_idx=qi,
                                      w_idx=wi, **kw, **common)
            else:
                r = oracle.layer_step(oracle.REUSE, idx_in=last_idx, **common)
            if mode in (I.FULL, I.REINDEX):
                last_idx = r.idx
            res.append(r)
        results[b] = res
        caches[b] = (kvc, kvs, ixc, ixs)
    return results, caches
