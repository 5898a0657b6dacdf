"""csa2_layer_step_static -- the layer step for callers that cannot allocate
-- against csa2_layer_step with a caller workspace: every layer's outputs
(Top-K indices, pool, attention output and lse) bit for bit, on two calls
in a row on the same GPU, the second with a smaller input (fewer sequences,
shorter context, smaller Top-K), so the static scratch holds the first
call's contents when the second starts.  A step needing more scratch than
the static array is rejected before anything is launched."""
import ctypes

import pytest
import torch

from sparse_attention_decode_e2m1_amd import api
from sparse_attention_decode_e2m1_amd import harness as Hn
from sparse_attention_decode_e2m1_amd import inputs as I

pytestmark = pytest.mark.gpu


def _outputs(dw):
    """Everything a layer writes: out and lse; idx_out for the layers that
    select (Full, Reindex); the pool of a Full layer that keeps one."""
    res = []
    for L in dw.layers:
        res.append([L.out.clone(), L.lse.clone()])
        if L.mode in (I.FULL, I.REINDEX):
            res[-1].append(L.idx_out.clone())
        if L.pool_out is not None:
            res[-1] += [L.pool_out.clone(), L.pool_count.clone()]
    return res


def _poison(dw):
    for L in dw.layers:
        L.idx_out.fill_(-7)
        L.out.fill_(float("nan"))
        L.lse.fill_(float("nan"))
        if L.pool_out is not None:
            L.pool_out.fill_(-7)
            L.pool_count.fill_(-7)


def _static_matches_workspace_step(w):
    dw = Hn.DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ref = _outputs(dw)
    _poison(dw)
    torch.cuda.synchronize()
    for li in range(len(dw.layers)):
        mode, args = dw._args[li]
        assert api.workspace_bytes(mode, args) <= api.STATIC_SCRATCH_BYTES
        api.layer_step_static(mode, args)
    torch.cuda.synchronize()
    got = _outputs(dw)
    for li, (a, b) in enumerate(zip(ref, got)):
        for x, y in zip(a, b):
            assert torch.equal(x, y), (w.name, li)


def test_static_scratch_step_twice_second_smaller():
    big = I.small("t_static_big", 66, B=4, N=40000, K=2048, P=4096,
                  modes=(I.FULL, I.REINDEX, I.REUSE, I.REUSE))
    small = I.small("t_static_small", 67, B=2, N=9000, K=256,
                    modes=(I.FULL, I.REINDEX, I.REUSE))
    print(f"[no-alloc] {big.name} then {small.name}", flush=True)
    _static_matches_workspace_step(big)
    _static_matches_workspace_step(small)


def test_static_scratch_rejects_a_step_beyond_its_size():
    w = I.WORKLOADS["C5_prefill_4k_on_128k"]
    F = ctypes.c_void_p(0x10000)  # never dereferenced: the size check comes first
    a = api.LayerArgs(B=1, T=w.T, H=16, D=576, dv=512, H_I=4, D_I=128, K=w.K, S=w.W - 1 + w.T,
                      W=w.W, sm_scale=0.04)
    a.kv = api.Fp4Cache(F, F, 576, w.N)
    a.icache = api.Fp4Cache(F, F, 128, w.N)
    for n in ("q", "q_pos", "swa", "swa_scale", "swa_pos0", "out", "idx_out", "q_idx", "w_idx",
              "new_kv", "new_ikey"):
        setattr(a, n, F)
    assert api.workspace_bytes(api.FULL, a) > api.STATIC_SCRATCH_BYTES
    st = api.raw_call("csa2_layer_step_static", api.FULL, ctypes.byref(a), None)
    assert st == 4
    assert b"static scratch" in api.lib().csa2_last_error()
