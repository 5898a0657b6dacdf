"""Device-side set-up and execution of a synthetic CSA2 layer group.

Builds the caches and per-layer inputs of a ``inputs.Workload`` on the GPU
(from the seeded host tensors of ``inputs``) and runs the group's layers in
order through ``api.layer_step``.  Wiring between layers follows the static
modes: a Reindex layer reuses the caches of the group's Full layer (and its
candidate pool when that layer kept one); a Reuse layer takes the Top-K
indices of the latest Full/Reindex layer; a window-only layer attends to its
window alone (Top-K 0).  Each Full layer starts a group with its own cache
set (identical contents: the caches come from the same seeded rows).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import api
from . import inputs as I


@dataclass
class LayerBuffers:
    mode: int
    q: torch.Tensor
    q_idx: torch.Tensor
    w_idx: torch.Tensor
    swa: torch.Tensor
    swa_scale: torch.Tensor
    swa_pos0: torch.Tensor
    idx_out: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor
    pool_out: Optional[torch.Tensor] = None
    pool_count: Optional[torch.Tensor] = None


class DeviceWorkload:
    """Caches (``copies`` identical sets per layer group, so a timed loop can
    rotate through more bytes than the 256 MB last-level cache holds) and
    layer buffers."""

    def __init__(self, w: I.Workload, copies: int = 1, device: str = "cuda",
                 seqs: Optional[List[int]] = None, reuse_one_launch: bool = False):
        self.w = w
        self.dev = device
        # Reuse and window-only layers through csa2_sparse_attn_one_launch
        # (the same attention, split and merge in one launch) instead of
        # csa2_layer_step
        self.reuse_one_launch = reuse_one_launch
        self._attn_kw = {}
        B, N, T = w.B, w.N, w.T
        self.rows = B * T
        # ---- caches: rows [0, ctx0) quantized at set-up, rows of the step
        # written by the Full layer.
        kvc = torch.zeros((B, N, w.D // 2), dtype=torch.uint8, device=device)
        kvs = torch.zeros((B, N, w.D // 16), dtype=torch.uint8, device=device)
        ixc = torch.zeros((B, N, w.DI // 2), dtype=torch.uint8, device=device)
        ixs = torch.zeros((B, N, w.DI // 16), dtype=torch.uint8, device=device)
        new_dtype = torch.bfloat16 if T > 1 else torch.float32
        self.new_kv = torch.empty((self.rows, w.D), dtype=new_dtype, device=device)
        self.new_ikey = torch.empty((self.rows, w.DI), dtype=new_dtype, device=device)
        for b in range(B):
            c = I.seq_cache(w, b)
            ctx0 = w.ctx0
            kv_b = c.kv[:ctx0].to(device)
            api.quantize_kv(kv_b, kvc[b, :ctx0], kvs[b, :ctx0])
            ik_b = c.ikey[:ctx0].to(device)
            api.quantize_kv(ik_b, ixc[b, :ctx0], ixs[b, :ctx0])
            self.new_kv[b * T:(b + 1) * T] = c.kv[ctx0:].to(new_dtype).to(device)
            self.new_ikey[b * T:(b + 1) * T] = c.ikey[ctx0:].to(new_dtype).to(device)
            del kv_b, ik_b, c
        torch.cuda.synchronize()
        self.group = I.group_of_layers(w.modes)
        self.ngroups = max(self.group) + 1
        self.rot = max(1, copies)  # rotation sets; set c, group g uses caches[c * ngroups + g]
        self.caches = [(kvc, kvs, ixc, ixs)]
        for _ in range(self.rot * self.ngroups - 1):
            self.caches.append(tuple(t.clone() for t in (kvc, kvs, ixc, ixs)))
        self.q_pos = torch.tensor([w.ctx0 + t for b in range(B) for t in range(T)],
                                  dtype=torch.int32, device=device)
        # ---- per-layer inputs and outputs
        self.layers: List[LayerBuffers] = []
        for li, mode in enumerate(w.modes):
            qs, qis, wis, swas, scs, p0s = [], [], [], [], [], []
            for b in range(B):
                L = I.layer_inputs(w, b, li)
                qs.append(L.q)
                qis.append(L.q_idx)
                wis.append(L.w_idx)
                swas.append(L.swa)
                scs.append(L.swa_scale)
                p0s.append(L.swa_pos0)
            has_pool = mode == I.FULL and w.P > 0
            K = 0 if mode == I.SWA else w.K
            self.layers.append(LayerBuffers(
                mode=mode,
                q=torch.cat(qs).contiguous().to(device),
                q_idx=torch.cat(qis).contiguous().to(device),
                w_idx=torch.cat(wis).contiguous().to(device),
                swa=torch.stack(swas).contiguous().to(device),
                swa_scale=torch.tensor(scs, dtype=torch.float32, device=device),
                swa_pos0=torch.tensor(p0s, dtype=torch.int32, device=device),
                idx_out=torch.full((self.rows, max(K, 1)), -1, dtype=torch.int32, device=device),
                out=torch.zeros((self.rows, w.H, w.DV), dtype=torch.float32, device=device),
                lse=torch.zeros((self.rows, w.H), dtype=torch.float32, device=device),
                pool_out=torch.full((self.rows, w.P), -1, dtype=torch.int32, device=device)
                if has_pool else None,
                pool_count=torch.zeros((self.rows,), dtype=torch.int32, device=device)
                if has_pool else None,
            ))
        self.S = self.layers[0].swa.shape[1]
        self._args = [self._layer_args(li, c) for c in range(self.rot)
                      for li in range(len(self.layers))]
        nbytes = max(api.workspace_bytes(a[0], a[1]) for a in self._args)
        for k in self._attn_kw.values():
            nbytes = max(nbytes, api.sparse_attn_workspace_bytes(w.B * w.T, k["K"], w.W, w.DV))
        self.ws = api.workspace(nbytes, device)
        torch.cuda.synchronize()

    # ------------------------------------------------------------------
    def _layer_args(self, li: int, copy: int):
        w = self.w
        kvc, kvs, ixc, ixs = self.caches[copy * self.ngroups + self.group[li]]
        L = self.layers[li]
        mode = L.mode
        src_idx = None
        pool_src = None
        for j in range(li - 1, -1, -1):
            if self.group[j] != self.group[li]:
                break
            m = self.layers[j].mode
            if src_idx is None and m in (I.FULL, I.REINDEX):
                src_idx = self.layers[j].idx_out
            if m == I.FULL and self.layers[j].pool_out is not None and pool_src is None:
                pool_src = self.layers[j]
        kw = dict(
            B=w.B, T=w.T, H=w.H, D=w.D, dv=w.DV, H_I=w.HI, D_I=w.DI,
            K=0 if mode == I.SWA else w.K,
            P=w.P if (mode == I.FULL) else 0, S=self.S, W=w.W, sm_scale=w.sm_scale,
            kv=api.cache(kvc, kvs, w.D, w.N), icache=api.cache(ixc, ixs, w.DI, w.N),
            q_pos=self.q_pos, q=L.q, swa=L.swa, swa_scale=L.swa_scale, swa_pos0=L.swa_pos0,
            out=L.out, lse=L.lse,
        )
        if mode == I.FULL:
            kw.update(new_kv=self.new_kv, new_ikey=self.new_ikey,
                      new_dtype=api.BF16 if self.new_kv.dtype == torch.bfloat16 else api.F32,
                      q_idx=L.q_idx, w_idx=L.w_idx, idx_out=L.idx_out,
                      pool_out=L.pool_out, pool_count_out=L.pool_count)
        elif mode == I.REINDEX:
            kw.update(q_idx=L.q_idx, w_idx=L.w_idx, idx_out=L.idx_out)
            if pool_src is not None:
                kw.update(pool_in=pool_src.pool_out, pool_count_in=pool_src.pool_count,
                          P_in=w.P)
        elif mode == I.REUSE:
            kw.update(idx_in=src_idx)
        if mode in (I.REUSE, I.SWA):
            self._attn_kw[(copy, li)] = dict(
                q=L.q, B=w.B, T=w.T, kv=kw["kv"], idx=src_idx if mode == I.REUSE else None,
                K=kw["K"], swa=L.swa, swa_scale=L.swa_scale, swa_pos0=L.swa_pos0, S=self.S,
                W=w.W, q_pos=self.q_pos, sm_scale=w.sm_scale, dv=w.DV, out=L.out, lse=L.lse)
        # a window-only layer is a Reuse call with no global entries
        return (I.REUSE if mode == I.SWA else mode), api.layer_args(**kw)

    def step(self, copy: int = 0, stream=None):
        """One pass of every layer of the group, in order."""
        for li in range(len(self.layers)):
            self.run_layer(li, copy, stream)

    def run_layer(self, li: int, copy: int = 0, stream=None):
        c = copy % self.rot
        if self.reuse_one_launch and (c, li) in self._attn_kw:
            k = self._attn_kw[(c, li)]
            api.sparse_attn_one_launch(k["q"], k["B"], k["T"], k["kv"], k["idx"], k["K"], k["swa"],
                                       k["swa_scale"], k["swa_pos0"], k["S"], k["W"], k["q_pos"],
                                       k["sm_scale"], k["dv"], k["out"], k["lse"], self.ws,
                                       stream=stream)
            return
        mode, args = self._args[c * len(self.layers) + li]
        api.layer_step(mode, args, self.ws, stream=stream)

    def cache_bytes(self):
        kvc, kvs, ixc, ixs = self.caches[0]
        return [t.clone() for t in (kvc, kvs, ixc, ixs)]
