"""The oracle over one sequence of a synthetic workload's layer group.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  Uses
the same seeded inputs as the device harness, the oracle's own FP4 caches
(quantized here from the fp32 source rows) and the same static wiring of
modes: Reindex searches the Full layer's caches (inside its pool when it kept
one); Reuse takes the latest Full/Reindex selection; a window-only layer
attends to its window alone.  Every group of the layer plan sees the same
cache contents (the device keeps one identical copy per group).
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from sparse_attention_decode_e2m1_amd import inputs as I

from . import FULL, REINDEX, REUSE, layer_step, quantize


class SeqGroup:
    def __init__(self, w: I.Workload, b: int, tokens: Optional[List[int]] = None):
        self.w, self.b = w, b
        self.tok = list(range(w.T)) if tokens is None else list(tokens)
        c = I.seq_cache(w, b)
        self.kv = c.kv.numpy()
        self.ik = c.ikey.numpy()
        kvc, kvs = quantize(self.kv[: w.ctx0])
        ixc, ixs = quantize(self.ik[: w.ctx0])
        # rows of the step start as zero bytes; the Full layer writes them
        self.kvc = np.concatenate([kvc, np.zeros((w.T, w.D // 2), np.uint8)])
        self.kvs = np.concatenate([kvs, np.zeros((w.T, w.D // 16), np.uint8)])
        self.ixc = np.concatenate([ixc, np.zeros((w.T, w.DI // 2), np.uint8)])
        self.ixs = np.concatenate([ixs, np.zeros((w.T, w.DI // 16), np.uint8)])
        self.all_pos = np.arange(w.ctx0, w.N)
        self.q_pos = self.all_pos[self.tok]
        self.layers = []
        for li in range(len(w.modes)):
            L = I.layer_inputs(w, b, li)
            self.layers.append(dict(
                q=L.q.float().numpy()[self.tok], q_idx=L.q_idx.float().numpy()[self.tok],
                w_idx=L.w_idx.numpy()[self.tok], swa=L.swa.numpy(), swa_scale=L.swa_scale,
                swa_pos0=L.swa_pos0))

    def step(self, keep_scores: bool = False):
        """Every layer of the group once; returns one LayerResult per layer."""
        w = self.w
        res = []
        last_idx = None
        pool = None
        for li, mode in enumerate(w.modes):
            L = self.layers[li]
            common = dict(q=L["q"], swa=L["swa"], swa_scale=L["swa_scale"],
                          swa_pos0=L["swa_pos0"], W=w.W, sm_scale=w.sm_scale, dv=w.DV, K=w.K,
                          kv_codes=self.kvc, kv_scales=self.kvs, q_pos=self.q_pos,
                          keep_scores=keep_scores)
            if mode == FULL:
                r = layer_step(FULL, ix_codes=self.ixc, ix_scales=self.ixs, q_idx=L["q_idx"],
                               w_idx=L["w_idx"], new_kv=self.kv[w.ctx0:],
                               new_ikey=self.ik[w.ctx0:], write_pos=self.all_pos, P=w.P,
                               **common)
                if w.P > 0:
                    pool = (r.pool, r.pool_count)
            elif mode == REINDEX:
                kw = {}
                if pool is not None:
                    kw = dict(pool_in=pool[0], pool_count_in=pool[1])
                r = layer_step(REINDEX, ix_codes=self.ixc, ix_scales=self.ixs,
                               q_idx=L["q_idx"], w_idx=L["w_idx"], **kw, **common)
            elif mode == I.SWA:
                # window-only layer: a Reuse call with no global entries
                common["K"] = 0
                r = layer_step(REUSE, idx_in=np.zeros((len(self.tok), 0), np.int32), **common)
            else:
                r = layer_step(REUSE, idx_in=last_idx, **common)
            if mode in (FULL, REINDEX):
                last_idx = r.idx
            res.append(r)
        return res

    def caches(self):
        return self.kvc, self.kvs, self.ixc, self.ixs
