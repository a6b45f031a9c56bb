"""Python binding of the gfx950 MSA hot-path library (libmsa_hip.so).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks dtype / device / contiguity, and forwards raw
pointers and sizes to the C ABI declared in include/msa.h.  Every step of the
computation runs in the HIP kernels of that library; there is no CPU or
PyTorch fallback, and importing the compute functions without the built
library raises.  Errors from the library are raised as MsaError carrying the
msa_status code.

Build the library in-tree first:  python -m block_sparse_attention_msa_amd.build

One decode step of an MSA layer (32 streams, one new token each):

    dims = msa_dims()                                   # 4 groups x 16 heads, top-16 of 128-key blocks
    cache = make_cache(k=k, v=v, idx_k=idx_k)           # [S][cap][4][128] bf16 / f32 tensors
    msa_index_append(dims, cache, stream, pos, max_pos, idx_k_new, k_new, v_new)
    msa_select(dims, cache, idx_q, stream, pos, max_pos, sel, n_sel,
               ws=torch.empty(workspace_bytes(dims, MSA_OP_SELECT, n_q, max_pos), dtype=torch.uint8, device="cuda"))
    msa_attend_decode(dims, cache, q, stream, pos, max_pos, sel, out, ws_attend)

A prefill chunk of one stream uses msa_select_prefill / msa_attend_prefill;
msa_index_project turns hidden states into idx_q and appends idx_k; the DSA
variant uses dsa_dims, dsa_index_append, dsa_select (or dsa_select_heads)
and dsa_attend_decode.  make_cache also describes paged caches (block_table),
an fp16 index cache (idx_k_f16) and int8 / 4-bit K/V (kv_format).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa_hip.so")

# msa_status
MSA_OK = 0
# msa_op
MSA_OP_SELECT = 1
MSA_OP_SELECT_PREFILL = 2
MSA_OP_ATTEND_DECODE = 3
MSA_OP_ATTEND_PREFILL = 4
DSA_OP_SELECT = 5
DSA_OP_ATTEND_DECODE = 6
MSA_OP_BLOCK_SCORES_PREFILL = 7
MSA_OP_INDEX_PROJECT = 8
MSA_OP_DECODE_STEP = 9
# call-size limits of include/msa.h
MSA_MAX_QUERIES = 1 << 18
MSA_MAX_ROWS = 1 << 24

EXPORTS = (
    "msa_workspace_bytes", "msa_status_string", "msa_index_append", "msa_block_scores",
    "msa_topk_blocks", "msa_select", "msa_block_scores_prefill", "msa_select_prefill",
    "msa_attend_decode", "msa_attend_prefill", "dsa_index_append", "dsa_select",
    "dsa_select_heads", "dsa_attend_decode", "msa_index_project", "msa_select_static",
    "msa_decode_step",
)


class MsaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


class Dims(ctypes.Structure):
    _fields_ = [("n_group", ctypes.c_int32), ("heads_per_group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("block", ctypes.c_int32), ("top_k", ctypes.c_int32), ("scale", ctypes.c_float)]


class Cache(ctypes.Structure):
    _fields_ = [("idx_k", ctypes.c_void_p), ("dsa_k", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("cap", ctypes.c_int64), ("n_stream", ctypes.c_int32),
                ("idx_k_f16", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("table_stride", ctypes.c_int32), ("kv_format", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


KV_BF16, KV_INT8, KV_Q4 = 0, 1, 2


class Proj(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("w_q", ctypes.c_void_p), ("w_k", ctypes.c_void_p),
                ("g_q", ctypes.c_void_p), ("g_k", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("rot_dim", ctypes.c_int32)]


def msa_dims(top_k: int = 16, scale: float = 128 ** -0.5) -> Dims:
    """The MiniMax-M3 sparse-layer geometry: 4 groups x 16 heads, d = 128,
    indexer d = 128, block 128."""
    return Dims(4, 16, 128, 128, 128, top_k, scale)


def dsa_dims(top_k: int = 2048, scale: float = 128 ** -0.5) -> Dims:
    """The DSA variant: token-granular selection (block 1) of top_k keys."""
    return Dims(4, 16, 128, 128, 1, top_k, scale)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_msa_amd.build` "
                "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        D, C = ctypes.POINTER(Dims), ctypes.POINTER(Cache)
        L.msa_workspace_bytes.argtypes = [D, ctypes.c_int, I64, I32]
        L.msa_workspace_bytes.restype = ctypes.c_size_t
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        sig = {
            "msa_index_append": [D, C, P, P, I64, I32, P, P, P, P],
            "dsa_index_append": [D, C, P, P, I64, I32, P, P, P, P],
            "msa_block_scores": [D, C, P, P, P, I64, I32, P, I64, P],
            "msa_topk_blocks": [D, P, I64, P, I64, I32, P, P, P],
            "msa_select": [D, C, P, P, P, I64, I32, P, P, P, ctypes.c_size_t, P],
            "msa_select_static": [D, C, P, P, P, I64, I32, P, P, P],
            "msa_block_scores_prefill": [D, C, P, I32, I32, I64, P, I64, P, ctypes.c_size_t, P],
            "msa_select_prefill": [D, C, P, I32, I32, I64, P, P, P, ctypes.c_size_t, P],
            "msa_attend_decode": [D, C, P, P, P, I64, I32, P, P, P, ctypes.c_size_t, P],
            "msa_attend_prefill": [D, C, P, I32, I32, I64, P, P, P, ctypes.c_size_t, P],
            "dsa_select": [D, C, P, P, P, I64, I32, P, P, P, ctypes.c_size_t, P],
            "dsa_select_heads": [D, C, P, P, I32, P, P, I64, I32, P, P, P, ctypes.c_size_t, P],
            "msa_index_project": [D, C, ctypes.POINTER(Proj), P, P, P, I64, I32, P, P, ctypes.c_size_t, P],
            "dsa_attend_decode": [D, C, P, P, P, I64, I32, P, P, P, ctypes.c_size_t, P],
            "msa_decode_step": [D, C, P, P, I64, I32, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().msa_status_string(code).decode()


def workspace_bytes(dims: Dims, op: int, n_q: int, max_pos: int) -> int:
    n = lib().msa_workspace_bytes(ctypes.byref(dims), op, n_q, max_pos)
    if n == ctypes.c_size_t(-1).value:
        raise MsaError(-6, "msa_workspace_bytes")
    return n


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _p(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(hip_stream) -> ctypes.c_void_p:
    if hip_stream is None:
        hip_stream = torch.cuda.current_stream()
    if isinstance(hip_stream, torch.cuda.Stream):
        hip_stream = hip_stream.cuda_stream
    return ctypes.c_void_p(int(hip_stream))


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    return _p(ws, name="ws"), ws.numel() * ws.element_size()


def _check(code: int, where: str):
    if code != MSA_OK:
        raise MsaError(code, where)


def make_cache(*, k: torch.Tensor, v: torch.Tensor, idx_k: Optional[torch.Tensor] = None,
               dsa_k: Optional[torch.Tensor] = None, idx_k_f16: Optional[torch.Tensor] = None,
               block_table: Optional[torch.Tensor] = None, cap: Optional[int] = None,
               kv_format: int = KV_BF16, k_scale: Optional[torch.Tensor] = None,
               v_scale: Optional[torch.Tensor] = None) -> Cache:
    """Cache descriptor over caller-owned tensors: k, v [S][cap][4][128] bf16;
    idx_k [S][cap][4][128] f32, or idx_k_f16 the same in f16; dsa_k
    [S][cap][128] f16.
    Paged: block_table [S][stride] int32 (page of each logical 128-token
    block), the caches pools [n_pages * 128][4][128] (dsa_k [n_pages * 128][128]),
    and cap the logical capacity per stream (<= stride * 128).
    Quantized K/V (kv_format KV_INT8 / KV_Q4): k, v uint8 codes [S][cap][4][128]
    (int8) or [S][cap][4][64] (two 4-bit codes per byte), k_scale, v_scale f32
    [S][cap][4][4] (one scale per 32 values); pools likewise when paged.
    The descriptor holds references to the tensors, so their memory stays
    allocated while it lives."""
    kv_dtype = torch.bfloat16 if kv_format == KV_BF16 else torch.uint8
    if kv_format != KV_BF16:
        width = 128 if kv_format == KV_INT8 else 64
        for name, t in (("k", k), ("v", v)):
            if t is not None and t.shape[-1] != width:
                raise ValueError(f"{name}: a kv_format {kv_format} cache holds {width} code bytes per group row")
        for name, t, ref in (("k_scale", k_scale, k), ("v_scale", v_scale, v)):
            if t is None or ref is None:
                continue
            if tuple(t.shape) != tuple(ref.shape[:-1]) + (4,):
                raise ValueError(f"{name}: expected shape {tuple(ref.shape[:-1]) + (4,)} (one f32 per 32 values)")
    if block_table is None:
        S, cap_ = k.shape[0], k.shape[1]
        table, stride = None, 0
    else:
        if cap is None:
            raise ValueError("a paged cache needs cap (positions per stream)")
        S, stride = block_table.shape
        cap_, table = cap, _p(block_table, torch.int32, "block_table")
    c = Cache(_p(idx_k, torch.float32, "idx_k"), _p(dsa_k, torch.float16, "dsa_k"),
              _p(k, kv_dtype, "k"), _p(v, kv_dtype, "v"), cap_, S,
              _p(idx_k_f16, torch.float16, "idx_k_f16"), table, stride, kv_format,
              _p(k_scale, torch.float32, "k_scale"), _p(v_scale, torch.float32, "v_scale"))
    c.tensors = (k, v, idx_k, dsa_k, idx_k_f16, block_table, k_scale, v_scale)
    return c


def make_proj(*, w_q: torch.Tensor, w_k: torch.Tensor, g_q: torch.Tensor, g_k: torch.Tensor,
              eps: float, rope_theta: float, rot_dim: int) -> Proj:
    """Indexer projection parameters over caller-owned f32 tensors: w_q, w_k
    [512][d_model], g_q, g_k [4][128]; held by reference while the
    descriptor lives."""
    if w_q.dim() != 2 or w_k.shape != w_q.shape:
        raise ValueError("w_q and w_k must be [512][d_model]")
    pr = Proj(w_q.shape[1], _p(w_q, torch.float32, "w_q"), _p(w_k, torch.float32, "w_k"),
              _p(g_q, torch.float32, "g_q"), _p(g_k, torch.float32, "g_k"), eps, rope_theta, rot_dim)
    pr.tensors = (w_q, w_k, g_q, g_k)
    return pr


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def msa_index_project(dims, cache, proj, x, stream, pos, max_pos, idx_q, ws, hip_stream=None):
    """x [n_tok][d_model] f32 -> idx_q [n_tok][4][128] f32; keys appended to the index cache."""
    wp, wn = _ws(ws)
    _check(lib().msa_index_project(ctypes.byref(dims), ctypes.byref(cache), ctypes.byref(proj),
                                   _p(x, torch.float32, "x"), _p(stream, torch.int32), _p(pos, torch.int32),
                                   pos.numel(), max_pos, _p(idx_q, torch.float32, "idx_q"), wp, wn,
                                   _stream(hip_stream)), "msa_index_project")


def msa_index_append(dims, cache, stream, pos, max_pos, idx_k_new=None, k_new=None, v_new=None,
                     hip_stream=None):
    _check(lib().msa_index_append(ctypes.byref(dims), ctypes.byref(cache), _p(stream, torch.int32),
                                  _p(pos, torch.int32), pos.numel(), max_pos,
                                  _p(idx_k_new, torch.float32, "idx_k_new"),
                                  _p(k_new, torch.bfloat16, "k_new"), _p(v_new, torch.bfloat16, "v_new"),
                                  _stream(hip_stream)), "msa_index_append")


def dsa_index_append(dims, cache, stream, pos, max_pos, key_new, k_new=None, v_new=None,
                     hip_stream=None):
    _check(lib().dsa_index_append(ctypes.byref(dims), ctypes.byref(cache), _p(stream, torch.int32),
                                  _p(pos, torch.int32), pos.numel(), max_pos,
                                  _p(key_new, torch.float16, "key_new"),
                                  _p(k_new, torch.bfloat16, "k_new"), _p(v_new, torch.bfloat16, "v_new"),
                                  _stream(hip_stream)), "dsa_index_append")


def msa_block_scores(dims, cache, idx_q, stream, pos, max_pos, bs, hip_stream=None):
    """bs: [n_q][4][nblk_stride] float32."""
    _check(lib().msa_block_scores(ctypes.byref(dims), ctypes.byref(cache), _p(idx_q, torch.float32),
                                  _p(stream, torch.int32), _p(pos, torch.int32), pos.numel(), max_pos,
                                  _p(bs, torch.float32, "bs"), bs.shape[-1], _stream(hip_stream)),
           "msa_block_scores")


def msa_topk_blocks(dims, bs, pos, max_pos, sel, n_sel, hip_stream=None):
    _check(lib().msa_topk_blocks(ctypes.byref(dims), _p(bs, torch.float32, "bs"), bs.shape[-1],
                                 _p(pos, torch.int32), pos.numel(), max_pos, _p(sel, torch.int32),
                                 _p(n_sel, torch.int32), _stream(hip_stream)), "msa_topk_blocks")


def msa_select(dims, cache, idx_q, stream, pos, max_pos, sel, n_sel, ws, hip_stream=None):
    wp, wn = _ws(ws)
    _check(lib().msa_select(ctypes.byref(dims), ctypes.byref(cache), _p(idx_q, torch.float32),
                            _p(stream, torch.int32), _p(pos, torch.int32), pos.numel(), max_pos,
                            _p(sel, torch.int32), _p(n_sel, torch.int32), wp, wn, _stream(hip_stream)),
           "msa_select")


def msa_select_static(dims, cache, idx_q, stream, pos, max_pos, sel, n_sel, hip_stream=None):
    """msa_select without a workspace: the block scores stay in the library's
    per-device array (MSA_STATIC_SCRATCH_BYTES); calls on one GPU must not
    overlap."""
    _check(lib().msa_select_static(ctypes.byref(dims), ctypes.byref(cache), _p(idx_q, torch.float32),
                                   _p(stream, torch.int32), _p(pos, torch.int32), pos.numel(), max_pos,
                                   _p(sel, torch.int32), _p(n_sel, torch.int32), _stream(hip_stream)),
           "msa_select_static")


MSA_STATIC_SCRATCH_BYTES = 4 << 20


def msa_block_scores_prefill(dims, cache, idx_q, stream_id, pos0, bs, ws, hip_stream=None):
    wp, wn = _ws(ws)
    _check(lib().msa_block_scores_prefill(ctypes.byref(dims), ctypes.byref(cache),
                                          _p(idx_q, torch.float32), stream_id, pos0, idx_q.shape[0],
                                          _p(bs, torch.float32, "bs"), bs.shape[-1], wp, wn,
                                          _stream(hip_stream)),
           "msa_block_scores_prefill")


def msa_select_prefill(dims, cache, idx_q, stream_id, pos0, sel, n_sel, ws, hip_stream=None):
    wp, wn = _ws(ws)
    _check(lib().msa_select_prefill(ctypes.byref(dims), ctypes.byref(cache), _p(idx_q, torch.float32),
                                    stream_id, pos0, idx_q.shape[0], _p(sel, torch.int32),
                                    _p(n_sel, torch.int32), wp, wn, _stream(hip_stream)),
           "msa_select_prefill")


def msa_attend_decode(dims, cache, q, stream, pos, max_pos, sel, out, ws=None, hip_stream=None):
    wp, wn = _ws(ws)
    _check(lib().msa_attend_decode(ctypes.byref(dims), ctypes.byref(cache), _p(q, torch.bfloat16, "q"),
                                   _p(stream, torch.int32), _p(pos, torch.int32), pos.numel(), max_pos,
                                   _p(sel, torch.int32), _p(out, torch.float32, "out"), wp, wn,
                                   _stream(hip_stream)), "msa_attend_decode")


def msa_decode_step(dims, cache, stream, pos, max_pos, idx_k_new, k_new, v_new, idx_q, q, sel, n_sel, out, ws,
                    hip_stream=None):
    """msa_index_append + msa_select + msa_attend_decode of one decode step
    (three kernels for few queries over short contexts)."""
    wp, wn = _ws(ws)
    _check(lib().msa_decode_step(ctypes.byref(dims), ctypes.byref(cache), _p(stream, torch.int32),
                                 _p(pos, torch.int32), pos.numel(), max_pos,
                                 _p(idx_k_new, torch.float32, "idx_k_new"), _p(k_new, torch.bfloat16, "k_new"),
                                 _p(v_new, torch.bfloat16, "v_new"), _p(idx_q, torch.float32, "idx_q"),
                                 _p(q, torch.bfloat16, "q"), _p(sel, torch.int32), _p(n_sel, torch.int32),
                                 _p(out, torch.float32, "out"), wp, wn, _stream(hip_stream)), "msa_decode_step")


def msa_attend_prefill(dims, cache, q, stream_id, pos0, sel, out, ws=None, hip_stream=None):
    wp, wn = _ws(ws)
    _check(lib().msa_attend_prefill(ctypes.byref(dims), ctypes.byref(cache), _p(q, torch.bfloat16, "q"),
                                    stream_id, pos0, q.shape[0], _p(sel, torch.int32),
                                    _p(out, torch.float32, "out"), wp, wn, _stream(hip_stream)),
           "msa_attend_prefill")


def dsa_select(dims, cache, q_idx, stream, pos, max_pos, sel, n_sel, ws, hip_stream=None):
    wp, wn = _ws(ws)
    _check(lib().dsa_select(ctypes.byref(dims), ctypes.byref(cache), _p(q_idx, torch.float16, "q_idx"),
                            _p(stream, torch.int32), _p(pos, torch.int32), pos.numel(), max_pos,
                            _p(sel, torch.int32), _p(n_sel, torch.int32), wp, wn, _stream(hip_stream)),
           "dsa_select")


def dsa_select_heads(dims, cache, q_idx_h, head_w, stream, pos, max_pos, sel, n_sel, ws, hip_stream=None):
    """q_idx_h [n_q][n_head][128] fp16, head_w [n_q][n_head] f32."""
    if q_idx_h.dim() != 3 or head_w.shape != q_idx_h.shape[:2]:
        raise ValueError("q_idx_h must be [n_q][n_head][128] and head_w [n_q][n_head]")
    wp, wn = _ws(ws)
    _check(lib().dsa_select_heads(ctypes.byref(dims), ctypes.byref(cache), _p(q_idx_h, torch.float16, "q_idx_h"),
                                  _p(head_w, torch.float32, "head_w"), q_idx_h.shape[1],
                                  _p(stream, torch.int32), _p(pos, torch.int32), pos.numel(), max_pos,
                                  _p(sel, torch.int32), _p(n_sel, torch.int32), wp, wn, _stream(hip_stream)),
           "dsa_select_heads")


def dsa_attend_decode(dims, cache, q, stream, pos, max_pos, sel, out, ws=None, hip_stream=None):
    wp, wn = _ws(ws)
    _check(lib().dsa_attend_decode(ctypes.byref(dims), ctypes.byref(cache), _p(q, torch.bfloat16, "q"),
                                   _p(stream, torch.int32), _p(pos, torch.int32), pos.numel(), max_pos,
                                   _p(sel, torch.int32), _p(out, torch.float32, "out"), wp, wn,
                                   _stream(hip_stream)), "dsa_attend_decode")
