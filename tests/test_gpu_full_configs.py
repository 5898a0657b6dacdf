"""GPU parity at the benchmark workloads' full sizes, through the same
csa2_layer_step launches the benchmark times (one cache copy), against the
oracle on the same seeded inputs: every query of the 4K, 64K batch-16,
256K group and 1M pool workloads, and a sample of the 4096 tokens of the
prefill chunk on 128K context (first, last and seeded random tokens; the
whole chunk is written and scored on the GPU)."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_e2m1_amd import harness as Hn
from sparse_attention_decode_e2m1_amd import inputs as I
from tests.gpu_common import compare_group, host
from tests.oracle_runner import run_group

pytestmark = pytest.mark.gpu


def run_and_compare(w, seqs=None, tokens=None):
    print(f"[full-size] {w.name}: B={w.B} N={w.N} T={w.T} K={w.K} P={w.P}", flush=True)
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ores, oc = run_group(w, seqs=seqs, tokens=tokens, keep_scores=True)
    return dw, compare_group(w, dw, ores, oc, seqs=seqs, tokens=tokens)


def test_c1_single_full_layer_4k():
    w = I.WORKLOADS["C1_full_4k"]
    _, same = run_and_compare(w)
    assert same >= 1


def test_c2_full_layer_batch16_64k():
    w = I.WORKLOADS["C2_full_b16_64k"]
    _, same = run_and_compare(w)
    assert same >= 12  # near-tie swaps at the K-th score are allowed, not common


def test_c3_group_batch4_256k():
    w = I.WORKLOADS["C3_group_b4_256k"]
    _, same = run_and_compare(w)
    assert same >= 6


def test_c4_pool_1m():
    w = I.WORKLOADS["C4_pool_1m"]
    dw, _ = run_and_compare(w)
    assert int(host(dw.layers[0].pool_count)[0]) == w.P
    # the Full layer's Top-K lies inside its pool
    assert set(host(dw.layers[0].idx_out)[0].tolist()) <= set(host(dw.layers[0].pool_out)[0].tolist())


def test_c5_prefill_chunk_sampled_tokens():
    w = I.WORKLOADS["C5_prefill_4k_on_128k"]
    rng = np.random.default_rng(5)
    tok = sorted({0, 1, 127, 128, w.T - 1} | set(rng.choice(w.T, 11, replace=False).tolist()))
    _, same = run_and_compare(w, tokens=tok)
    assert same >= len(tok) // 2
