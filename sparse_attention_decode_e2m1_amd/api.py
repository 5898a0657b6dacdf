"""ctypes binding of libcsa2.so (argument marshalling only).

Every function takes torch tensors that live on the GPU, passes their device
pointers to the C ABI declared in ``include/csa2.h`` and raises on a non-OK
status.  All computation happens in the library's HIP kernels; if the library
is missing this module raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("CSA2_LIB") or os.path.join(HERE, "libcsa2.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "csa2.h")

FULL, REINDEX, REUSE = 0, 1, 2
F32, BF16 = 0, 1
HEADS = 16
ERR_INCOMPLETE = 7
# csa2_topk_variant
TOPK_AUTO, TOPK_ROW, TOPK_ONE_WAIT, TOPK_SELECT, TOPK_SELECT_CUT, TOPK_SELECT_LARGE, \
    TOPK_SELECT_LARGE_CUT, TOPK_SAMPLED, TOPK_SAMPLED_FALLBACK, TOPK_BAND, TOPK_BAND_EXACT = range(11)
TOPK_LIST_FINISH = 16

c_i32, c_i64, c_f32, c_p, c_sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                  ctypes.c_void_p, ctypes.c_size_t)


class Fp4Cache(ctypes.Structure):
    _fields_ = [("codes", c_p), ("scales", c_p), ("dim", c_i32), ("cap", c_i64)]


class Fp8Cache(ctypes.Structure):
    _fields_ = [("codes", c_p), ("scales", c_p), ("dim", c_i32), ("cap", c_i64)]


class LayerArgs(ctypes.Structure):
    _fields_ = [
        ("B", c_i32), ("T", c_i32), ("H", c_i32), ("D", c_i32), ("dv", c_i32),
        ("H_I", c_i32), ("D_I", c_i32), ("K", c_i32), ("P", c_i32), ("S", c_i32), ("W", c_i32),
        ("sm_scale", c_f32),
        ("kv", Fp4Cache), ("icache", Fp4Cache),
        ("q_pos", c_p), ("new_kv", c_p), ("new_ikey", c_p), ("new_dtype", c_i32),
        ("q", c_p), ("q_idx", c_p), ("w_idx", c_p),
        ("swa", c_p), ("swa_scale", c_p), ("swa_pos0", c_p),
        ("idx_in", c_p), ("idx_out", c_p),
        ("pool_in", c_p), ("pool_count_in", c_p), ("P_in", c_i32),
        ("pool_out", c_p), ("pool_count_out", c_p),
        ("out", c_p), ("lse", c_p),
    ]


class Csa2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"csa2 status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libcsa2.so (built in-tree by ``build.py``); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_decode_e2m1_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "csa2_quantize_kv": (c_i32, [c_p, c_i32, c_i64, c_i32, c_i64, c_p, c_p, c_p, c_p]),
            "csa2_rope_quantize_kv": (c_i32, [c_p, c_i32, c_i64, c_i32, c_i64, c_i32, c_p, c_p,
                                              c_p, c_p, c_p]),
            "csa2_quantize_kv_fp8": (c_i32, [c_p, c_i32, c_i64, c_i32, c_i64, c_p, c_p, c_p, c_p]),
            "csa2_sparse_attn_fp8": (c_i32, [c_p, c_i32, c_i32, c_i32, ctypes.POINTER(Fp8Cache),
                                             c_p, c_i32, c_p, c_p, c_p, c_i32, c_i32, c_p, c_f32,
                                             c_i32, c_p, c_p, c_p, c_sz, c_p]),
            "csa2_index_score": (c_i32, [ctypes.POINTER(Fp4Cache), c_i32, c_i32, c_p, c_p, c_i32,
                                         c_p, c_p, c_i32, c_i64, c_p, c_p]),
            "csa2_topk_workspace_bytes": (c_sz, [c_i32, c_i64, c_i32]),
            "csa2_topk": (c_i32, [c_p, c_i32, c_i64, c_p, c_p, c_i32, c_p, c_p, c_p, c_sz, c_p]),
            "csa2_sparse_attn_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32]),
            "csa2_sparse_attn": (c_i32, [c_p, c_i32, c_i32, c_i32, ctypes.POINTER(Fp4Cache), c_p,
                                         c_i32, c_p, c_p, c_p, c_i32, c_i32, c_p, c_f32, c_i32,
                                         c_p, c_p, c_p, c_sz, c_p]),
            "csa2_sparse_attn_one_launch": (c_i32, [c_p, c_i32, c_i32, c_i32,
                                                    ctypes.POINTER(Fp4Cache), c_p, c_i32, c_p,
                                                    c_p, c_p, c_i32, c_i32, c_p, c_f32, c_i32,
                                                    c_p, c_p, c_p, c_sz, c_p]),
            "csa2_workspace_bytes": (c_sz, [c_i32, ctypes.POINTER(LayerArgs)]),
            "csa2_layer_step": (c_i32, [c_i32, ctypes.POINTER(LayerArgs), c_p, c_sz, c_p]),
            "csa2_fp4_bytes_per_token": (c_i64, [c_i32]),
            "csa2_workspace_init": (c_i32, [c_p, c_sz, c_p]),
            "csa2_status_string": (ctypes.c_char_p, [c_i32]),
            "csa2_last_error": (ctypes.c_char_p, []),
            "csa2_version": (ctypes.c_char_p, []),
            "csa2_layer_args_size": (c_sz, []),
            "csa2_fp4_cache_size": (c_sz, []),
            "csa2_workspace_control_bytes": (c_sz, [c_i32]),
            "csa2_profile_begin": (c_i32, []),
            "csa2_profile_end": (c_i32, [ctypes.POINTER(c_i32), ctypes.POINTER(ctypes.c_double)]),
            "csa2_workspace_check": (c_i32, [c_p, c_sz, c_i32, c_p]),
            "csa2_layer_step_static": (c_i32, [c_i32, ctypes.POINTER(LayerArgs), c_p]),
            "csa2_stream_read": (c_i32, [c_p, c_sz, c_p, c_i32, c_p]),
            "csa2_set_topk_variant": (c_i32, [c_i32]),
            "csa2_topk_last_variant": (c_i32, []),
            "csa2_set_wait_limit": (ctypes.c_uint32, [ctypes.c_uint32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        if (L.csa2_layer_args_size() != ctypes.sizeof(LayerArgs)
                or L.csa2_fp4_cache_size() != ctypes.sizeof(Fp4Cache)):
            raise ImportError("csa2_layer_args / csa2_fp4_cache layout mismatch with libcsa2.so")
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/csa2.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def _check(status: int):
    if status != 0:
        L = lib()
        raise Csa2Error(status, f"{L.csa2_status_string(status).decode()}: "
                                f"{L.csa2_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "tensors must be contiguous GPU tensors"
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _bf16_bits(t: torch.Tensor) -> torch.Tensor:
    assert t.dtype == torch.bfloat16
    return t


def cache(codes: torch.Tensor, scales: torch.Tensor, dim: int, cap: int) -> Fp4Cache:
    """Cache descriptor; it holds references to its tensors so their device
    memory stays allocated as long as the descriptor is used."""
    c = Fp4Cache(_ptr(codes), _ptr(scales), dim, cap)
    c._keep = (codes, scales)
    return c


# ------------------------------------------------------------------ wrappers
def fp4_bytes_per_token(dim: int) -> int:
    return int(lib().csa2_fp4_bytes_per_token(dim))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (filled by the library's kernel)."""
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    _check(lib().csa2_workspace_init(_ptr(ws), ws.numel(), _stream()))
    return ws


def quantize_kv(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                dst_rows: Optional[torch.Tensor] = None, stream=None):
    dt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    rows, dim = x.shape
    _check(lib().csa2_quantize_kv(_ptr(x), dt, rows, dim, x.stride(0), _ptr(dst_rows),
                                  _ptr(codes), _ptr(scales), _stream(stream)))


def rope_quantize_kv(x: torch.Tensor, rope_dim: int, cos_sin: Optional[torch.Tensor],
                     codes: torch.Tensor, scales: torch.Tensor,
                     dst_rows: Optional[torch.Tensor] = None, stream=None):
    """csa2_rope_quantize_kv: rotary pairs of the last rope_dim channels
    rotated by cos_sin [rows][rope_dim/2][2] (fp32), then quantize-on-write."""
    dt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    rows, dim = x.shape
    _check(lib().csa2_rope_quantize_kv(_ptr(x), dt, rows, dim, x.stride(0), rope_dim,
                                       _ptr(cos_sin), _ptr(dst_rows), _ptr(codes), _ptr(scales),
                                       _stream(stream)))


def index_score(icache: Fp4Cache, B: int, T: int, q_idx: torch.Tensor, w: torch.Tensor,
                n_valid: torch.Tensor, scores: torch.Tensor, pool: Optional[torch.Tensor] = None,
                stream=None):
    HI = q_idx.shape[-2]
    P = pool.shape[-1] if pool is not None else 0
    _check(lib().csa2_index_score(ctypes.byref(icache), B, T, _ptr(_bf16_bits(q_idx)), _ptr(w), HI,
                                  _ptr(n_valid), _ptr(pool), P, scores.shape[-1], _ptr(scores),
                                  _stream(stream)))


def topk_workspace_bytes(rows: int, n: int, k: int) -> int:
    return int(lib().csa2_topk_workspace_bytes(rows, n, k))


def topk(scores: torch.Tensor, n_valid: torch.Tensor, k: int, idx_out: torch.Tensor,
         ws: torch.Tensor, slot_pos: Optional[torch.Tensor] = None,
         count_out: Optional[torch.Tensor] = None, stream=None):
    rows, n = scores.shape
    _check(lib().csa2_topk(_ptr(scores), rows, n, _ptr(n_valid), _ptr(slot_pos), k, _ptr(idx_out),
                           _ptr(count_out), _ptr(ws), ws.numel(), _stream(stream)))


def sparse_attn_workspace_bytes(rows: int, K: int, W: int, dv: int) -> int:
    return int(lib().csa2_sparse_attn_workspace_bytes(rows, K, W, dv))


def sparse_attn(q: torch.Tensor, B: int, T: int, kv: Fp4Cache, idx: Optional[torch.Tensor],
                K: int, swa: Optional[torch.Tensor], swa_scale: Optional[torch.Tensor],
                swa_pos0: Optional[torch.Tensor], S: int, W: int, q_pos: torch.Tensor,
                sm_scale: float, dv: int, out: torch.Tensor, lse: Optional[torch.Tensor],
                ws: torch.Tensor, stream=None):
    H = q.shape[-2]
    _check(lib().csa2_sparse_attn(_ptr(_bf16_bits(q)), B, T, H, ctypes.byref(kv), _ptr(idx), K,
                                  _ptr(swa), _ptr(swa_scale), _ptr(swa_pos0), S, W, _ptr(q_pos),
                                  float(sm_scale), dv, _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                  _stream(stream)))


def sparse_attn_one_launch(q: torch.Tensor, B: int, T: int, kv: Fp4Cache,
                           idx: Optional[torch.Tensor], K: int, swa: Optional[torch.Tensor],
                           swa_scale: Optional[torch.Tensor], swa_pos0: Optional[torch.Tensor],
                           S: int, W: int, q_pos: torch.Tensor, sm_scale: float, dv: int,
                           out: torch.Tensor, lse: Optional[torch.Tensor], ws: torch.Tensor,
                           stream=None):
    H = q.shape[-2]
    _check(lib().csa2_sparse_attn_one_launch(_ptr(_bf16_bits(q)), B, T, H, ctypes.byref(kv),
                                             _ptr(idx), K, _ptr(swa), _ptr(swa_scale),
                                             _ptr(swa_pos0), S, W, _ptr(q_pos), float(sm_scale),
                                             dv, _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                             _stream(stream)))


def fp8_cache(codes: torch.Tensor, scales: torch.Tensor, dim: int, cap: int) -> Fp8Cache:
    """Descriptor of an FP8 main cache: codes [B][cap][dim] u8, scales [B][cap]
    f32; like cache(), it keeps its tensors alive."""
    c = Fp8Cache(_ptr(codes), _ptr(scales), dim, cap)
    c._keep = (codes, scales)
    return c


def quantize_kv_fp8(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                    dst_rows: Optional[torch.Tensor] = None, stream=None):
    dt = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    rows, dim = x.shape
    _check(lib().csa2_quantize_kv_fp8(_ptr(x), dt, rows, dim, x.stride(0), _ptr(dst_rows),
                                      _ptr(codes), _ptr(scales), _stream(stream)))


def sparse_attn_fp8(q: torch.Tensor, B: int, T: int, kv: Fp8Cache, idx: Optional[torch.Tensor],
                    K: int, swa: Optional[torch.Tensor], swa_scale: Optional[torch.Tensor],
                    swa_pos0: Optional[torch.Tensor], S: int, W: int, q_pos: torch.Tensor,
                    sm_scale: float, dv: int, out: torch.Tensor, lse: Optional[torch.Tensor],
                    ws: torch.Tensor, stream=None):
    H = q.shape[-2]
    _check(lib().csa2_sparse_attn_fp8(_ptr(_bf16_bits(q)), B, T, H, ctypes.byref(kv), _ptr(idx), K,
                                      _ptr(swa), _ptr(swa_scale), _ptr(swa_pos0), S, W,
                                      _ptr(q_pos), float(sm_scale), dv, _ptr(out), _ptr(lse),
                                      _ptr(ws), ws.numel(), _stream(stream)))


def layer_args(**kw) -> LayerArgs:
    """Build csa2_layer_args from keyword arguments (tensors or ints)."""
    a = LayerArgs()
    keep = []
    for name, _ in LayerArgs._fields_:
        if name not in kw or kw[name] is None:
            continue
        v = kw[name]
        keep.append(v)  # device memory referenced by pointer stays alive with `a`
        if isinstance(v, torch.Tensor):
            setattr(a, name, _ptr(v))
        else:
            setattr(a, name, v)
    a._keep = keep
    return a


def workspace_bytes(mode: int, args: LayerArgs) -> int:
    return int(lib().csa2_workspace_bytes(mode, ctypes.byref(args)))


def layer_step(mode: int, args: LayerArgs, ws: torch.Tensor, stream=None):
    _check(lib().csa2_layer_step(mode, ctypes.byref(args), _ptr(ws), ws.numel(), _stream(stream)))


STATIC_SCRATCH_BYTES = 64 << 20


def layer_step_static(mode: int, args: LayerArgs, stream=None):
    """csa2_layer_step_static: the layer step with the library's static
    scratch as its workspace (no allocation in the call)."""
    _check(lib().csa2_layer_step_static(mode, ctypes.byref(args), _stream(stream)))


PROFILE_KERNELS = ("quantize", "index_score", "topk_select", "sparse_attn", "pool_gather")


def profile_begin():
    _check(lib().csa2_profile_begin())


def profile_end() -> dict:
    """{kernel: (launches, summed event time in ms)} since profile_begin()."""
    n = len(PROFILE_KERNELS)
    counts = (c_i32 * n)()
    tot = (ctypes.c_double * n)()
    _check(lib().csa2_profile_end(counts, tot))
    return {k: (int(counts[i]), float(tot[i])) for i, k in enumerate(PROFILE_KERNELS)}


def workspace_check(ws: torch.Tensor, rows: int, stream=None):
    """csa2_workspace_check: raises Csa2Error (status ERR_INCOMPLETE) if a
    one-wait launch on this workspace gave up waiting."""
    _check(lib().csa2_workspace_check(_ptr(ws), ws.numel(), rows, _stream(stream)))


def stream_read(src: torch.Tensor, sink: torch.Tensor, blocks: int, stream=None):
    """csa2_stream_read: a plain streaming read of src (the HBM reference)."""
    _check(lib().csa2_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), blocks,
                                  _stream(stream)))


def set_topk_variant(variant: int) -> int:
    """Force a Top-K variant (TOPK_*); returns the previous setting."""
    return int(lib().csa2_set_topk_variant(variant))


def topk_last_variant() -> int:
    return int(lib().csa2_topk_last_variant())


def set_wait_limit(polls: int) -> int:
    return int(lib().csa2_set_wait_limit(polls))


def raw_call(name: str, *args):
    """Call an entry point with raw ctypes arguments; returns its status."""
    return getattr(lib(), name)(*args)
