"""GPU parity at the benchmark workloads' full sizes, through the same
csa2_layer_step launches the benchmark times (one cache copy), against the
oracle on the same seeded inputs: every query of the 4K, 64K batch-16,
256K group and 1M pool workloads, and a 64-token sample of the 4096 tokens
of the prefill chunk on 128K context (first, last and seeded random tokens;
the whole chunk is written, scored, selected and attended on the GPU).
Every (sequence, layer, token) row's attention is compared."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_e2m1_amd import harness as Hn
from sparse_attention_decode_e2m1_amd import inputs as I
from tests.gpu_common import compare_group, expected_rows, host
from tests.oracle_runner import run_group

pytestmark = pytest.mark.gpu


def run_and_compare(w, seqs=None, tokens=None):
    print(f"[full-size] {w.name}: B={w.B} N={w.N} T={w.T} K={w.K} P={w.P}", flush=True)
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ores, oc = run_group(w, seqs=seqs, tokens=tokens, keep_scores=True)
    chk = compare_group(w, dw, ores, oc, seqs=seqs, tokens=tokens)
    print(f"[full-size] {w.name}: {chk}", flush=True)
    assert chk.rows == expected_rows(w, seqs, tokens)
    return dw, chk


def test_c1_single_full_layer_4k():
    w = I.WORKLOADS["C1_full_4k"]
    _, chk = run_and_compare(w)
    assert chk.same_sets >= 1


def test_c2_full_layer_batch16_64k():
    w = I.WORKLOADS["C2_full_b16_64k"]
    _, chk = run_and_compare(w)
    assert chk.same_sets >= 12  # near-tie swaps at the K-th score are allowed, not common


def test_c3_group_batch4_256k():
    w = I.WORKLOADS["C3_group_b4_256k"]
    _, chk = run_and_compare(w)
    assert chk.same_sets >= 6


def test_c4_pool_1m():
    w = I.WORKLOADS["C4_pool_1m"]
    dw, chk = run_and_compare(w)
    assert chk.pools == 1 and chk.rows == 3
    assert int(host(dw.layers[0].pool_count)[0]) == w.P
    # the Full layer's Top-K lies inside its pool
    assert set(host(dw.layers[0].idx_out)[0].tolist()) <= set(host(dw.layers[0].pool_out)[0].tolist())


def test_c5_prefill_chunk_sampled_tokens():
    w = I.WORKLOADS["C5_prefill_4k_on_128k"]
    rng = np.random.default_rng(5)
    # the first and last tokens, and those around the 2048-row pass and the
    # 1024-row attention launch boundaries
    fixed = {0, 1, 1023, 1024, 2047, 2048, 3071, 3072, w.T - 2, w.T - 1}
    rest = [t for t in rng.permutation(w.T).tolist() if t not in fixed][: 64 - len(fixed)]
    tok = sorted(fixed | set(rest))
    assert len(tok) == 64
    _, chk = run_and_compare(w, tokens=tok)
    assert chk.same_sets >= len(tok) // 2
