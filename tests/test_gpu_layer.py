"""GPU parity of csa2_layer_step (Full / Reindex / Reuse, pool, prefill) on
reduced workloads with the structure of the benchmark's, against the oracle
run on the same seeded inputs."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_e2m1_amd import api
from sparse_attention_decode_e2m1_amd import harness as Hn
from sparse_attention_decode_e2m1_amd import inputs as I
from tests.gpu_common import compare_group, host
from tests.oracle_runner import run_group

pytestmark = pytest.mark.gpu


def test_group_decode_small():
    w = I.small("t_group", 60, B=2, N=20000, K=512, modes=(I.FULL, I.REINDEX, I.REUSE, I.REUSE))
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ores, oc = run_group(w, keep_scores=True)
    assert compare_group(w, dw, ores, oc) >= 3


def test_group_reuse_layers_in_one_launch():
    """The decode group with its Reuse layers run by the one-launch attention
    gives every layer's output and lse bit for bit as csa2_layer_step does."""
    w = I.small("t_group1", 62, B=4, N=20000, K=2048,
                modes=(I.FULL, I.REINDEX, I.REUSE, I.REUSE))
    ref = Hn.DeviceWorkload(w)
    ref.step()
    one = Hn.DeviceWorkload(w, reuse_one_launch=True)
    for _ in range(2):
        one.step()
    torch.cuda.synchronize()
    for a, b in zip(ref.layers, one.layers):
        assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)
    words = one.ws[: api.lib().csa2_workspace_control_bytes(w.B * w.T)].view(torch.int32)
    assert int(torch.count_nonzero(words)) == 0


def test_group_pool_small():
    w = I.small("t_pool", 61, B=1, N=60000, K=512, P=4096,
                modes=(I.FULL, I.REINDEX, I.REINDEX), salient=True)
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    assert int(host(dw.layers[0].pool_count)[0]) == 4096
    idx0 = set(host(dw.layers[0].idx_out)[0].tolist())
    assert idx0 <= set(host(dw.layers[0].pool_out)[0].tolist())
    ores, oc = run_group(w, keep_scores=True)
    compare_group(w, dw, ores, oc)


def test_pool_larger_than_context_equals_flat():
    """P >= n: the pool is every position and Top-K equals the flat result."""
    wp = I.small("t_poolbig", 62, B=1, N=3000, K=256, P=4096, modes=(I.FULL,))
    wf = I.small("t_poolbig", 62, B=1, N=3000, K=256, P=0, modes=(I.FULL,))
    a, b = Hn.DeviceWorkload(wp), Hn.DeviceWorkload(wf)
    a.step()
    b.step()
    torch.cuda.synchronize()
    assert int(host(a.layers[0].pool_count)[0]) == 3000
    assert list(host(a.layers[0].pool_out)[0][:3000]) == list(range(3000))
    assert (host(a.layers[0].pool_out)[0][3000:] == -1).all()
    assert np.array_equal(host(a.layers[0].idx_out), host(b.layers[0].idx_out))
    assert np.array_equal(host(a.layers[0].out), host(b.layers[0].out))


def test_prefill_small():
    w = I.small("t_prefill", 63, B=1, N=5000, T=64, K=256, modes=(I.FULL,))
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ores, oc = run_group(w, keep_scores=True)
    assert compare_group(w, dw, ores, oc) >= 32


def test_reuse_and_reindex_reproduce_full_on_gpu():
    """A Reuse layer fed the Full layer's indices, query and window gives the
    Full output bit for bit; a Reindex layer fed the Full layer's indexer
    query selects the same indices."""
    w = I.small("t_repro", 64, B=2, N=9000, K=300, modes=(I.FULL, I.REINDEX, I.REUSE))
    dw = Hn.DeviceWorkload(w)
    F = dw.layers[0]
    dw.layers[1].q_idx.copy_(F.q_idx)
    dw.layers[1].w_idx.copy_(F.w_idx)
    dw.step()
    torch.cuda.synchronize()
    assert torch.equal(dw.layers[1].idx_out, F.idx_out)
    kvc, kvs, ixc, ixs = dw.caches[0]
    out = torch.zeros_like(F.out)
    lse = torch.zeros_like(F.lse)
    args = api.layer_args(B=w.B, T=w.T, H=16, D=576, dv=512, H_I=4, D_I=128, K=w.K, S=dw.S,
                          W=w.W, sm_scale=w.sm_scale, kv=api.cache(kvc, kvs, 576, w.N),
                          q_pos=dw.q_pos, q=F.q, swa=F.swa, swa_scale=F.swa_scale,
                          swa_pos0=F.swa_pos0, idx_in=F.idx_out, out=out, lse=lse)
    api.layer_step(api.REUSE, args, dw.ws)
    torch.cuda.synchronize()
    assert torch.equal(out, F.out) and torch.equal(lse, F.lse)


def test_step_is_deterministic_and_leaves_workspace_clean():
    w = I.small("t_det", 65, B=2, N=30000, K=1024, modes=(I.FULL, I.REINDEX, I.REUSE))
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    first = [(L.idx_out.clone(), L.out.clone(), L.lse.clone()) for L in dw.layers]
    for _ in range(3):
        dw.step()
    torch.cuda.synchronize()
    for L, (i0, o0, l0) in zip(dw.layers, first):
        assert torch.equal(L.idx_out, i0) and torch.equal(L.out, o0) and torch.equal(L.lse, l0)
    ctl = dw.ws[: api.lib().csa2_workspace_control_bytes(dw.rows)].view(torch.int32)
    assert int(torch.count_nonzero(ctl)) == 0


def test_forty_layer_plan_small():
    """The 40-layer static plan (2 window-only layers, then 4 groups of Full,
    Reindex and Reuse layers, each group over its own cache copy) against the
    oracle, layer by layer."""
    w = I.small("t_forty", 64, B=1, N=3000, K=256, modes=I.forty_layer_modes())
    dw = Hn.DeviceWorkload(w)
    assert dw.ngroups == 4 and len(dw.caches) == 4
    dw.step()
    torch.cuda.synchronize()
    ores, oc = run_group(w, keep_scores=True)
    assert compare_group(w, dw, ores, oc) >= 6
    ctl = dw.ws[: api.lib().csa2_workspace_control_bytes(dw.rows)].view(torch.int32)
    assert int(torch.count_nonzero(ctl)) == 0

