"""Runs the oracle over a synthetic workload's layer group (test
infrastructure); see oracle.group."""
from __future__ import annotations

from typing import List, Optional

from oracle.group import SeqGroup
from sparse_attention_decode_e2m1_amd import inputs as I


def run_group(w: I.Workload, seqs: Optional[List[int]] = None,
              tokens: Optional[List[int]] = None, keep_scores: bool = False):
    """Returns {b: [LayerResult per layer]} and {b: oracle caches after the step}."""
    seqs = list(range(w.B)) if seqs is None else seqs
    results, caches = {}, {}
    for b in seqs:
        g = SeqGroup(w, b, tokens)
        results[b] = g.step(keep_scores=keep_scores)
        caches[b] = g.caches()
    return results, caches
