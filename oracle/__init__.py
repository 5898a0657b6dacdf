"""Plain CPU oracle for the CSA2 compressed-sparse-attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the GPU library (``sparse_attention_decode_e2m1_amd``); the only module
both sides use is the seeded input generator, which holds none of the method's
arithmetic.

The primitives live in ``csa2_oracle.c`` (double precision, plain
definitions); this module loads them through ctypes and composes the
per-layer modes from them.  Pages cited:

* [P1] helmcode.com/deepseek-v41-flash
* [P4] louisbouchard.ai/deepseek-v41-flash-kv-cache-writing-benchmark
* [P5] 0x0moeen.in/writes/deepseek-v4-1-flash-kv-cache
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcsa2_oracle.so")
_lib = None

FULL, REINDEX, REUSE = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain IEEE double arithmetic, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.csa2o_e2m1_value.argtypes, L.csa2o_e2m1_value.restype = [ctypes.c_int], f64
        L.csa2o_e4m3_value.argtypes, L.csa2o_e4m3_value.restype = [ctypes.c_int], f64
        L.csa2o_scale_byte.argtypes, L.csa2o_scale_byte.restype = [f64], ctypes.c_int
        L.csa2o_e2m1_code.argtypes, L.csa2o_e2m1_code.restype = [f64, f64], ctypes.c_int
        L.csa2o_quantize_rows.argtypes = [P, i64, i32, P, P]
        L.csa2o_quantize_rows.restype = None
        L.csa2o_dequant_rows.argtypes = [P, P, i64, i32, P]
        L.csa2o_dequant_rows.restype = None
        L.csa2o_index_score.argtypes = [P, P, i32, P, P, i32, P, i64, P]
        L.csa2o_index_score.restype = None
        L.csa2o_topk.argtypes = [P, i64, i32, P, P]
        L.csa2o_topk.restype = i32
        L.csa2o_sparse_attn.argtypes = [P, i32, i32, i32, P, P, P, i32, P, f64, i32, f64, P, P]
        L.csa2o_sparse_attn.restype = None
        L.csa2o_num_threads.argtypes, L.csa2o_num_threads.restype = [], i32
        L.csa2o_set_num_threads.argtypes, L.csa2o_set_num_threads.restype = [i32], None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().csa2o_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (timing only)."""
    lib().csa2o_set_num_threads(int(n))


# ---------------------------------------------------------------- codec
def e2m1_value(code: int) -> float:
    return lib().csa2o_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().csa2o_e4m3_value(int(byte))


def scale_byte(amax: float) -> int:
    return lib().csa2o_scale_byte(float(amax))


def e2m1_code(x: float, s: float) -> int:
    return lib().csa2o_e2m1_code(float(x), float(s))


def quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """[P1 §04 FP4]: E2M1 codes with one E4M3 scale per 16 channels, scale
    = amax/6, no global scale.  x: [rows][dim] values (fp32 or exactly
    representable in fp32).  Returns codes [rows][dim/2], scales [rows][dim/16]."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    rows, dim = x.shape
    assert dim % 16 == 0
    assert np.isfinite(x).all(), "non-finite inputs are unsupported"
    codes = np.empty((rows, dim // 2), np.uint8)
    scales = np.empty((rows, dim // 16), np.uint8)
    lib().csa2o_quantize_rows(_p(x), rows, dim, _p(codes), _p(scales))
    return codes, scales


def quantize_fp8(x) -> tuple[np.ndarray, np.ndarray]:
    """FP8 variant of the main cache ([P1 §04]: V4 Flash stored its global
    KV in FP8; the pages give no scale layout, read here as one fp32 scale
    per row).  scale = amax/448 over the row (1 for an all-zero row), both
    in IEEE float32; bytes = E4M3 of clamp(x/scale, -448, 448) in float32,
    rounded to nearest even (torch's float8_e4m3fn cast is that rounding).
    Returns bytes [rows][dim] u8 and scales [rows] f32."""
    import torch
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    assert np.isfinite(x).all(), "non-finite inputs are unsupported"
    amax = np.abs(x).max(axis=1)
    sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / sc[:, None], np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    b = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(b), sc


def e4m3_decode(b) -> np.ndarray:
    """E4M3 bytes to their values (float64) through the oracle's own table."""
    table = np.array([e4m3_value(v & 0x7F) * (-1.0 if v & 0x80 else 1.0) for v in range(256)])
    return table[np.asarray(b, dtype=np.uint8)]


def sparse_attn_fp8(q: np.ndarray, codes: np.ndarray, scales: np.ndarray, idx: np.ndarray,
                    wrows: np.ndarray, swa_scale: float, sm_scale: float, dv: int):
    """Sparse attention over an FP8 main cache, as the plain definition in
    float64: the selected rows (entries < 0 skipped) decoded as
    e4m3(byte) * scale[row], the window rows as e4m3(byte) * swa_scale, one
    softmax over their concatenation ([P4 "Share the cache and the search
    work"]), values = the first dv channels.  Returns out [H][dv], lse [H]."""
    q = np.asarray(q, dtype=np.float64)
    sel = np.asarray(idx, dtype=np.int64)
    sel = sel[sel >= 0]
    rows = e4m3_decode(codes[sel]) * np.asarray(scales, np.float64)[sel][:, None]
    if len(wrows):
        rows = np.concatenate([rows, e4m3_decode(wrows) * float(swa_scale)])
    H = q.shape[0]
    if len(rows) == 0:
        return np.zeros((H, dv)), np.full(H, -np.inf)
    logits = (q @ rows.T) * float(sm_scale)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ rows[:, :dv]) / l, (m + np.log(l))[:, 0]


def rope_rotate(x, cos_sin, rope_dim: int) -> np.ndarray:
    """Rotary pairs of the last rope_dim channels ([P1 §04]: the FP4
    quantisation is applied after RoPE; the pages give no rotary parameters,
    so the per-pair (cos, sin) come in as inputs).  Pair i = channels
    (dim - rope_dim + 2i, +1): y0 = x0 c - x1 s, y1 = x0 s + x1 c, written in
    float32 with every product and every sum rounded on its own (numpy's
    float32 arithmetic: no fused multiply-add).  x: [rows][dim];
    cos_sin: [rows][rope_dim/2][2]."""
    x = np.array(x, dtype=np.float32, copy=True)
    if rope_dim == 0:
        return x
    cs = np.asarray(cos_sin, dtype=np.float32)
    c, sn = cs[..., 0], cs[..., 1]
    base = x.shape[1] - rope_dim
    x0 = x[:, base::2].copy()
    x1 = x[:, base + 1::2].copy()
    x[:, base::2] = (x0 * c) - (x1 * sn)
    x[:, base + 1::2] = (x0 * sn) + (x1 * c)
    return x


def rope_quantize(x, cos_sin, rope_dim: int) -> tuple[np.ndarray, np.ndarray]:
    """Quantize-on-write after the rotary step: quantize(rope_rotate(x))."""
    return quantize(rope_rotate(x, cos_sin, rope_dim))


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    out = np.empty((rows, half * 2), np.float64)
    lib().csa2o_dequant_rows(_p(codes), _p(scales), rows, half * 2, _p(out))
    return out


def bytes_per_token(dim: int) -> int:
    """Stored bytes of one FP4 row: dim/2 code bytes + dim/16 scale bytes."""
    return dim // 2 + dim // 16


# ---------------------------------------------------------------- indexer
def index_scores(icodes: np.ndarray, iscales: np.ndarray, q: np.ndarray,
                 w: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Score = sum_h w_h * relu(q_h . k_row) for each listed cache row of one
    sequence ([P1 §03 CSA2]: a Reindex layer scores positions with its own
    query; the exact formula is a reading of the pages)."""
    icodes = np.ascontiguousarray(icodes, np.uint8)
    iscales = np.ascontiguousarray(iscales, np.uint8)
    q = np.ascontiguousarray(q, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    rows = np.ascontiguousarray(rows, np.int64)
    H, dim = q.shape
    out = np.empty(rows.shape[0], np.float64)
    lib().csa2o_index_score(_p(icodes), _p(iscales), dim, _p(q), _p(w), H,
                            _p(rows), rows.shape[0], _p(out))
    return out


# ---------------------------------------------------------------- top-k
def topk(scores: np.ndarray, n_valid: int, k: int,
         slot_pos: Optional[np.ndarray] = None) -> tuple[np.ndarray, int]:
    """[P4 "Share the cache and the search work"]: select k entries.  Order
    by score descending then slot ascending; output ascending, -1 padded."""
    scores = np.ascontiguousarray(scores, np.float64)
    assert np.isfinite(scores[:n_valid]).all()
    out = np.empty(k, np.int32)
    sp = None
    if slot_pos is not None:
        slot_pos = np.ascontiguousarray(slot_pos, np.int32)
        sp = _p(slot_pos)
    n = lib().csa2o_topk(_p(scores), int(n_valid), int(k), sp, _p(out))
    return out, int(n)


# ---------------------------------------------------------------- attention
def sparse_attn(q: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                idx: np.ndarray, swa: np.ndarray, swa_scale: float,
                sm_scale: float, dv: int) -> tuple[np.ndarray, np.ndarray]:
    """[P4 "Share the cache and the search work"]: attention over the selected
    global entries alongside the local window; one softmax over the union.
    q: [H][D]; codes/scales: one sequence's main cache; swa: the visible
    window rows [S][D] (E4M3 bytes)."""
    q = np.ascontiguousarray(q, np.float32)
    H, D = q.shape
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    idx = np.ascontiguousarray(idx, np.int32)
    swa = np.ascontiguousarray(swa, np.uint8).reshape(-1, D)
    out = np.empty((H, dv), np.float64)
    lse = np.empty(H, np.float64)
    lib().csa2o_sparse_attn(_p(q), H, D, dv, _p(codes), _p(scales), _p(idx),
                            idx.shape[0], _p(swa), float(swa_scale), swa.shape[0],
                            float(sm_scale), _p(out), _p(lse))
    return out, lse


def window_rows(swa: np.ndarray, swa_pos0: int, p: int, W: int) -> np.ndarray:
    """Rows of a window array (row r holds position swa_pos0 + r) visible to
    a query at position p: positions [p-W+1, p] present in the array."""
    lo = max(p - W + 1, swa_pos0)
    hi = min(p, swa_pos0 + swa.shape[0] - 1)
    if hi < lo:
        return swa[:0]
    return swa[lo - swa_pos0: hi - swa_pos0 + 1]


# ---------------------------------------------------------------- layer modes
@dataclass
class LayerResult:
    out: np.ndarray          # [T][H][dv]
    lse: np.ndarray          # [T][H]
    idx: np.ndarray          # [T][K] selected positions (ascending, -1 pad)
    scores: Optional[list] = None   # per token: scores over the scored list
    pool: Optional[np.ndarray] = None        # [T][P] (FULL with a pool)
    pool_count: Optional[np.ndarray] = None  # [T]


def layer_step(mode: int, *, q, swa, swa_scale, swa_pos0, W, sm_scale, dv, K,
               kv_codes, kv_scales, q_pos, ix_codes=None, ix_scales=None,
               q_idx=None, w_idx=None, new_kv=None, new_ikey=None,
               idx_in=None, P: int = 0, pool_in=None, pool_count_in=None,
               keep_scores: bool = False, write_pos=None) -> LayerResult:
    """One CSA2 layer for one sequence ([P1 §03 CSA2]; [P5 "Then every layer
    stops asking the same question"]: static Full / Reindex / Reuse modes).

    FULL writes the T new rows (main and index) at positions q_pos, scores
    every visible position, selects (through a pool of P when P > 0) and
    attends.  REINDEX scores the referenced caches with its own indexer
    query (inside pool_in when given).  REUSE attends over idx_in.  The
    caches passed in are modified in place by FULL (the write is part of
    the step).  Positions visible to token t: [0, q_pos[t]].  ``write_pos``
    (default q_pos) lists the rows FULL writes, so a sample of a prefill
    chunk's tokens can be evaluated after the whole chunk is written."""
    q = np.asarray(q, np.float32)
    T = q.shape[0]
    H = q.shape[1]
    out = np.zeros((T, H, dv))
    lse = np.zeros((T, H))
    idx_all = np.full((T, K), -1, np.int32)
    pools = np.full((T, P), -1, np.int32) if (mode == FULL and P > 0) else None
    pool_counts = np.zeros(T, np.int32) if pools is not None else None
    kept = [] if keep_scores else None
    if mode == FULL:
        wp = q_pos if write_pos is None else write_pos
        nc, ns = quantize(new_kv)
        kv_codes[wp] = nc
        kv_scales[wp] = ns
        ic, iS = quantize(new_ikey)
        ix_codes[wp] = ic
        ix_scales[wp] = iS
    for t in range(T):
        p = int(q_pos[t])
        if mode in (FULL, REINDEX):
            if mode == REINDEX and pool_in is not None:
                cnt = int(pool_count_in[t])
                slots = np.asarray(pool_in[t][:cnt], np.int64)
                sc = index_scores(ix_codes, ix_scales, q_idx[t], w_idx[t], slots)
                idx, _ = topk(sc, cnt, K, slot_pos=np.asarray(pool_in[t], np.int32))
            else:
                rows = np.arange(p + 1, dtype=np.int64)
                sc = index_scores(ix_codes, ix_scales, q_idx[t], w_idx[t], rows)
                if mode == FULL and P > 0:
                    pool, cnt = topk(sc, p + 1, P)
                    pools[t] = pool
                    pool_counts[t] = cnt
                    idx, _ = topk(sc[pool[:cnt]], cnt, K, slot_pos=pool)
                else:
                    idx, _ = topk(sc, p + 1, K)
            if kept is not None:
                kept.append(sc)
        else:
            idx = np.asarray(idx_in[t], np.int32)
        idx_all[t] = idx
        wrows = window_rows(np.asarray(swa), int(swa_pos0), p, W)
        o, l = sparse_attn(q[t], kv_codes, kv_scales, idx, wrows, swa_scale,
                           sm_scale, dv)
        out[t] = o
        lse[t] = l
    return LayerResult(out, lse, idx_all, kept, pools, pool_counts)
