"""GPU parity of csa2_layer_step (Full / Reindex / Reuse, pool, prefill) on
reduced workloads with the structure of the benchmark's, against the oracle
run on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle

from sparse_attention_decode_e2m1_amd import api
from sparse_attention_decode_e2m1_amd import harness as Hn
from sparse_attention_decode_e2m1_amd import inputs as I
from tests.gpu_common import compare_group, expected_rows, host
from tests.oracle_runner import run_group

pytestmark = pytest.mark.gpu


def test_group_decode_small():
    w = I.small("t_group", 60, B=2, N=20000, K=512, modes=(I.FULL, I.REINDEX, I.REUSE, I.REUSE))
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ores, oc = run_group(w, keep_scores=True)
    chk = compare_group(w, dw, ores, oc)
    assert chk.rows == expected_rows(w) and chk.same_sets >= 3


def test_group_decode_context_shorter_than_k():
    """Contexts of fewer positions than K: every visible position is kept,
    the rest of each index row is -1, and the attention skips the padding."""
    w = I.small("t_short", 59, B=2, N=150, K=256, modes=(I.FULL, I.REINDEX, I.REUSE))
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    for li in (0, 1):
        idx = host(dw.layers[li].idx_out)
        for row in idx:
            nv = w.N  # decode: the query sits at position N - 1 and sees [0, N)
            assert list(row[:nv]) == list(range(nv)) and (row[nv:] == -1).all()
    ores, oc = run_group(w, keep_scores=True)
    chk = compare_group(w, dw, ores, oc)
    assert chk.rows == expected_rows(w)


@pytest.mark.parametrize("hi", [1, 2])
def test_group_decode_fewer_index_heads(hi):
    """A decode group whose indexer has 1 or 2 heads (the scan packs more
    tiles per MFMA) against the oracle."""
    w = I.small(f"t_group_hi{hi}", 66 + hi, B=2, N=20000, K=512, modes=(I.FULL, I.REINDEX, I.REUSE),
                HI=hi)
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ores, oc = run_group(w, keep_scores=True)
    chk = compare_group(w, dw, ores, oc)
    assert chk.rows == expected_rows(w) and chk.same_sets >= 3


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


@pytest.mark.parametrize("P,B", [(4096, 1), (12000, 2)])
def test_group_pool_small(P, B):
    """Pools of 4096 slots and of 12000 (whose selections keep the keys in
    registers), one and two sequences."""
    w = I.small("t_pool", 61, B=B, N=60000, K=512, P=P,
                modes=(I.FULL, I.REINDEX, I.REINDEX), salient=True)
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    assert (host(dw.layers[0].pool_count) == P).all()
    for b in range(B):
        idx0 = set(host(dw.layers[0].idx_out)[b].tolist())
        assert idx0 <= set(host(dw.layers[0].pool_out)[b].tolist())
    ores, oc = run_group(w, keep_scores=True)
    chk = compare_group(w, dw, ores, oc)
    assert chk.rows == expected_rows(w) and chk.pools == B


@pytest.mark.parametrize("N,P", [(3000, 4096), (10000, 12000)])
def test_pool_larger_than_context_equals_flat(N, P):
    """P >= n: the pool is every position (the rest of the pool row -1) and
    Top-K equals the flat result."""
    wp = I.small("t_poolbig", 62, B=1, N=N, K=256, P=P, modes=(I.FULL,))
    wf = I.small("t_poolbig", 62, B=1, N=N, K=256, P=0, modes=(I.FULL,))
    a, b = Hn.DeviceWorkload(wp), Hn.DeviceWorkload(wf)
    a.step()
    b.step()
    torch.cuda.synchronize()
    assert int(host(a.layers[0].pool_count)[0]) == N
    assert list(host(a.layers[0].pool_out)[0][:N]) == list(range(N))
    assert (host(a.layers[0].pool_out)[0][N:] == -1).all()
    assert np.array_equal(host(a.layers[0].idx_out), host(b.layers[0].idx_out))
    assert np.array_equal(host(a.layers[0].out), host(b.layers[0].out))


def test_prefill_small():
    w = I.small("t_prefill", 63, B=1, N=5000, T=64, K=256, modes=(I.FULL,))
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ores, oc = run_group(w, keep_scores=True)
    chk = compare_group(w, dw, ores, oc)
    assert chk.rows == expected_rows(w) and chk.same_sets >= 32


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
    chk = compare_group(w, dw, ores, oc)
    assert chk.rows == expected_rows(w) and chk.same_sets >= 6
    ctl = dw.ws[: api.lib().csa2_workspace_control_bytes(dw.rows)].view(torch.int32)
    assert int(torch.count_nonzero(ctl)) == 0



def _edge_rows(rows, dim, seed):
    """Rows whose 16-channel blocks sit on rounding boundaries: blocks with
    amax exactly on a scale threshold (6 x the halfway point between E4M3
    neighbours, or an fp32 neighbour of it) and blocks whose elements lie
    exactly on the E2M1 halfway points of an E4M3 scale."""
    rng = np.random.default_rng(seed)
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = (e4[:-1] + e4[1:]) / 2
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    x = np.zeros((rows, dim), np.float32)
    for r in range(rows):
        for k in range(dim // 16):
            n = seed + r * (dim // 16) + k
            blk = np.empty(16, np.float32)
            if n % 2 == 0:
                j = (n // 2 * 5) % 126
                blk[:] = rng.standard_normal(16) * 0.1 * mids[j]
                a = np.float32(6 * mids[j])
                a = [a, np.nextafter(a, np.float32(np.inf)), np.nextafter(a, np.float32(0))][n % 3]
                blk[rng.integers(16)] = a if n % 4 else -a
            else:
                s = e4[(n * 11) % 127]
                blk[:] = np.concatenate([t, -t])[rng.permutation(16)] * s
            x[r, 16 * k:16 * k + 16] = blk
    return x


@pytest.mark.parametrize("new_dtype,hi", [("f32", 4), ("bf16", 4), ("f32_edges", 4), ("f32", 2),
                                          ("f32", 1)])
def test_full_decode_writes_and_scores_the_new_rows(new_dtype, hi):
    """A Full decode step writes its new rows inside the scan launch: the
    written rows equal the oracle's quantization of the new rows bit for bit,
    and the layer's score row (left in the workspace: it follows the control
    block) equals the oracle's indexer scores at every visible position,
    the new one included, within the fp32 accumulation bound.  The edge
    variant puts every block of the new rows on a rounding boundary; 1 and 2
    indexer heads take the same fused write."""
    w = I.small("t_fresh", 68, B=3, N=7000, K=256, modes=(I.FULL,), HI=hi)
    dw = Hn.DeviceWorkload(w)
    if new_dtype == "bf16":
        dw.new_kv = dw.new_kv.to(torch.bfloat16)
        dw.new_ikey = dw.new_ikey.to(torch.bfloat16)
        dw._args = [dw._layer_args(0, 0)]
    elif new_dtype == "f32_edges":
        dw.new_kv.copy_(torch.from_numpy(_edge_rows(w.B, dw.new_kv.shape[-1], 3)).view_as(dw.new_kv))
        dw.new_ikey.copy_(torch.from_numpy(_edge_rows(w.B, dw.new_ikey.shape[-1], 4)).view_as(dw.new_ikey))
    dw.step()
    torch.cuda.synchronize()
    kvc, kvs, ixc, ixs = (host(t) for t in dw.caches[0])
    p = w.N - 1
    nkv = dw.new_kv.float().cpu().numpy()
    nik = dw.new_ikey.float().cpu().numpy()
    off = api.lib().csa2_workspace_control_bytes(w.B)
    sc = host(dw.ws[off: off + w.B * w.N * 4].view(torch.float32).view(w.B, w.N))
    L = dw.layers[0]
    for b in range(w.B):
        c, s = oracle.quantize(nkv[b:b + 1])
        assert np.array_equal(kvc[b, p], c[0]) and np.array_equal(kvs[b, p], s[0]), b
        c, s = oracle.quantize(nik[b:b + 1])
        assert np.array_equal(ixc[b, p], c[0]) and np.array_equal(ixs[b, p], s[0]), b
        q = L.q_idx[b].float().cpu().numpy()
        wi = L.w_idx[b].cpu().numpy()
        rows = np.arange(w.N, dtype=np.int64)
        o = oracle.index_scores(ixc[b], ixs[b], q, wi, rows)
        k = oracle.dequant(ixc[b], ixs[b])
        bound = (np.abs(k) @ np.abs(q.astype(np.float64)).T * np.abs(wi.astype(np.float64))).sum(1)
        err = np.abs(sc[b] - o)
        assert (err <= 1e-5 * bound + 1e-30).all(), (b, int(err.argmax()), err.max())
        assert abs(sc[b, p] - o[p]) <= 1e-5 * bound[p] + 1e-30


def test_cache_save_and_reload_reproduces_the_step(tmp_path):
    """Checkpoint and resume of the persistent global cache (helmcode.com/
    deepseek-v41-flash, section "05 · cache hierarchy": the global KV is kept
    for later reuse): the FP4 planes of both caches are written to files and
    read back into a fresh set of caches (zeroed first).  Every layer that
    reads them -- Reindex scoring and selection, Reuse attention -- gives
    bit-identical indices, outputs and lse."""
    w = I.small("t_ckpt", 69, B=2, N=20000, K=512, modes=(I.FULL, I.REINDEX, I.REUSE))
    a = Hn.DeviceWorkload(w)
    a.step()
    torch.cuda.synchronize()
    names = ("kv_codes", "kv_scales", "ix_codes", "ix_scales")
    for n, t in zip(names, a.caches[0]):
        np.save(tmp_path / f"{n}.npy", host(t))
    b = Hn.DeviceWorkload(w)
    for t in b.caches[0]:
        t.zero_()
    for n, t in zip(names, b.caches[0]):
        t.copy_(torch.from_numpy(np.load(tmp_path / f"{n}.npy")))
    for li in (1, 2):  # Reindex and Reuse read only the reloaded caches
        b.run_layer(li)
    torch.cuda.synchronize()
    for x, y in zip(a.caches[0], b.caches[0]):
        assert torch.equal(x, y)
    for li in (1, 2):
        La, Lb = a.layers[li], b.layers[li]
        if La.mode == I.REINDEX:
            assert torch.equal(La.idx_out, Lb.idx_out), li
        assert torch.equal(La.out, Lb.out) and torch.equal(La.lse, Lb.lse), li
