"""fp64 CPU oracle of the MSA hot path and the DSA lightning-indexer variant.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
the two share no code.  The arithmetic lives in ``msa_oracle.c`` (plain C,
fp64, one OpenMP loop over independent (query, group) items); this module only
compiles it with gcc and marshals numpy arrays through ctypes.

Sources, by page title and section:
  * "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support" (llama.cpp pull
    request 24908): Overview, Implementation, Limitations, review thread.
  * llama.cpp compare page b10146, commit "mtmd: Add Vision Support for
    Minimax-M3 (#25113)" (the squashed MSA history).
  * "deepseek2 : GLM-DSA sparse attention (lightning indexer), --dsa off by
    default" (ik_llama.cpp pull request 2045): What this does.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
            "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double


def _declare(L):
    L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_f64.restype = _D
    L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_f16_to_f64.restype = _D
    L.oracle_f64_to_f16_rne.argtypes = [_D]
    L.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
    L.oracle_select_ranked.argtypes = [_P, _I64, _I64, _I, _P]
    L.oracle_select_ranked.restype = _I
    L.oracle_msa_select.argtypes = [_I, _I, _I, _I, _I64, _P, _I64, _P, _P, _P,
                                    _P, _I64, _P, _P]
    L.oracle_msa_select.restype = _I
    L.oracle_sparse_attend.argtypes = [_I, _I, _I, _D, _I64, _P, _P, _I64, _P, _P,
                                       _P, _P, _I64, _I64, _I, _I, _P]
    L.oracle_sparse_attend.restype = _I
    L.oracle_dsa_rotate.argtypes = [_I64, _I, _P, _P]
    L.oracle_dsa_rotate.restype = _I
    L.oracle_dsa_select.argtypes = [_I, _I, _I64, _P, _I64, _P, _P, _P, _P, _P, _P]
    L.oracle_dsa_select.restype = _I
    L.oracle_dsa_select_heads.argtypes = [_I, _I, _I, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P]
    L.oracle_dsa_select_heads.restype = _I
    L.oracle_index_project.argtypes = [_I64, _I, _I, _I, _P, _P, _P, _P, _P, _D, _D, _I, _P, _P, _P]
    L.oracle_index_project.restype = _I
    L.oracle_kv_quantize.argtypes = [_I64, _I, _I, _P, _P, _P]
    L.oracle_kv_quantize.restype = _I
    L.oracle_kv_dequantize.argtypes = [_I64, _I, _I, _P, _P, _P]
    L.oracle_kv_dequantize.restype = _I
    L.oracle_sparse_attend_f64.argtypes = [_I, _I, _I, _D, _I64, _P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _I, _I, _P]
    L.oracle_sparse_attend_f64.restype = _I


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _idx(a) -> np.ndarray:
    """Index arrays (streams, positions, ids) are marshalled to int32."""
    return np.ascontiguousarray(np.asarray(a), np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# Conversions (exposed for their own pins)
# ---------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    f = lib().oracle_bf16_to_f64
    return np.array([f(int(b)) for b in np.asarray(bits, np.uint16).ravel()]).reshape(np.shape(bits))


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    f = lib().oracle_f16_to_f64
    return np.array([f(int(b)) for b in np.asarray(bits, np.uint16).ravel()]).reshape(np.shape(bits))


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    f = lib().oracle_f64_to_f16_rne
    return np.array([f(float(v)) for v in np.asarray(x, np.float64).ravel()],
                    dtype=np.uint16).reshape(np.shape(x))


# ---------------------------------------------------------------------------
# MSA
# ---------------------------------------------------------------------------
def select_ranked(score: np.ndarray, local: int, top_k: int) -> np.ndarray:
    """Rank candidates (local first, then score desc, id asc); ascending ids of
    the first min(top_k, n), padded with -1."""
    score = _c(score, np.float64)
    sel = np.empty(top_k, np.int32)
    lib().oracle_select_ranked(_ptr(score), score.size, local, top_k, _ptr(sel))
    return sel


def msa_select(idx_k, stream, pos, idx_q, *, block=128, top_k=16, nblk_out=None):
    """Block scores and top-k block selection.

    idx_k: [S][cap][G][Di] f32; stream, pos: [n_q] int32; idx_q: [n_q][G][Di].
    Returns (bs [n_q][G][nblk_out] f64, sel [n_q][G][top_k] i32, n_sel [n_q][G]).
    """
    idx_k = _c(idx_k, np.float32)
    idx_q = _c(idx_q, np.float32)
    stream = _idx(stream)
    pos = _idx(pos)
    _, cap, G, Di = idx_k.shape
    n_q = pos.size
    if nblk_out is None:
        nblk_out = (int(pos.max()) // block + 1) if n_q else 0
    bs = np.empty((n_q, G, nblk_out), np.float64)
    sel = np.empty((n_q, G, top_k), np.int32)
    n_sel = np.empty((n_q, G), np.int32)
    rc = lib().oracle_msa_select(G, Di, block, top_k, cap, _ptr(idx_k), n_q,
                                 _ptr(stream), _ptr(pos), _ptr(idx_q), _ptr(bs),
                                 nblk_out, _ptr(sel), _ptr(n_sel))
    if rc != 0:
        raise ValueError(f"oracle_msa_select failed: {rc}")
    return bs, sel, n_sel


def sparse_attend(k_cache, v_cache, stream, pos, q, sel, *, unit, scale,
                  heads_per_group=16, shared_across_groups=False):
    """Softmax attention of every query head over its group's selected units.

    k_cache, v_cache: [S][cap][G][D] bf16 bit patterns (uint16);
    q: [n_q][G*Hg][D] uint16 (bf16 bits); sel: [n_q][G][L] (or [n_q][L] when
    shared_across_groups).  Returns out [n_q][G*Hg][D] float64.
    """
    k_cache = _c(k_cache, np.uint16)
    v_cache = _c(v_cache, np.uint16)
    q = _c(q, np.uint16)
    sel = _idx(sel)
    stream = _idx(stream)
    pos = _idx(pos)
    _, cap, G, D = k_cache.shape
    n_q = pos.size
    if shared_across_groups:
        L = sel.shape[-1]
        q_stride, g_stride = L, 0
    else:
        L = sel.shape[-1]
        q_stride, g_stride = G * L, L
    out = np.empty((n_q, G * heads_per_group, D), np.float64)
    rc = lib().oracle_sparse_attend(G, heads_per_group, D, float(scale), cap,
                                    _ptr(k_cache), _ptr(v_cache), n_q, _ptr(stream),
                                    _ptr(pos), _ptr(q), _ptr(sel), q_stride, g_stride,
                                    L, unit, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_sparse_attend failed: {rc}")
    return out


# ---------------------------------------------------------------------------
# DSA
# ---------------------------------------------------------------------------
def dsa_rotate(k_raw: np.ndarray) -> np.ndarray:
    """fp16 rows [..., n] -> fp16_rne(H_n x / sqrt(n)) as uint16 bits."""
    k_raw = _c(k_raw, np.uint16)
    n = k_raw.shape[-1]
    out = np.empty_like(k_raw)
    rc = lib().oracle_dsa_rotate(k_raw.size // n, n, _ptr(k_raw), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dsa_rotate: row length must be a power of two")
    return out


def dsa_select(k_rot, stream, pos, q_idx, *, top_k=2048, want_scores=False):
    """k_rot: [S][cap][Di] fp16 bits; q_idx: [n_q][Di] fp16 bits.

    Returns (sel [n_q][top_k], n_sel [n_q], scores [n_q][cap] or None)."""
    k_rot = _c(k_rot, np.uint16)
    q_idx = _c(q_idx, np.uint16)
    stream = _idx(stream)
    pos = _idx(pos)
    _, cap, Di = k_rot.shape
    n_q = pos.size
    scores = np.empty((n_q, cap), np.float64) if want_scores else None
    sel = np.empty((n_q, top_k), np.int32)
    n_sel = np.empty(n_q, np.int32)
    rc = lib().oracle_dsa_select(Di, top_k, cap, _ptr(k_rot), n_q, _ptr(stream),
                                 _ptr(pos), _ptr(q_idx), _ptr(scores), _ptr(sel),
                                 _ptr(n_sel))
    if rc != 0:
        raise ValueError(f"oracle_dsa_select failed: {rc}")
    return sel, n_sel, scores


def dsa_select_heads(k_rot, stream, pos, q_idx_h, head_w, *, top_k=2048, want_scores=False):
    """Multi-head lightning indexer: score(i, j) = sum_h w[i][h] *
    max(0, q[i][h] . k[j]) (the reduction is a reading: the DSA pull request's
    review thread gives per-head scores, an element-wise product and a head
    reduction, not the formula), then the same top-k as dsa_select.

    k_rot: [S][cap][Di] fp16 bits; q_idx_h: [n_q][H][Di] fp16 bits;
    head_w: [n_q][H] f32.  Returns (sel, n_sel, scores or None)."""
    k_rot = _c(k_rot, np.uint16)
    q_idx_h = _c(q_idx_h, np.uint16)
    head_w = _c(head_w, np.float32)
    stream = _idx(stream)
    pos = _idx(pos)
    _, cap, Di = k_rot.shape
    n_q, H = head_w.shape
    if q_idx_h.shape != (n_q, H, Di):
        raise ValueError("q_idx_h must be [n_q][H][Di]")
    scores = np.empty((n_q, cap), np.float64) if want_scores else None
    sel = np.empty((n_q, top_k), np.int32)
    n_sel = np.empty(n_q, np.int32)
    rc = lib().oracle_dsa_select_heads(Di, H, top_k, cap, _ptr(k_rot), n_q, _ptr(stream), _ptr(pos),
                                       _ptr(q_idx_h), _ptr(head_w), _ptr(scores), _ptr(sel), _ptr(n_sel))
    if rc != 0:
        raise ValueError(f"oracle_dsa_select_heads failed: {rc}")
    return sel, n_sel, scores


def index_project(x, w_q, w_k, g_q, g_k, pos, *, eps, theta, rot_dim, n_group=4, want_q=True, want_k=True):
    """Indexer projection: per token and group, y = W x, gemma-style RMS norm
    (times 1 + gamma), RoPE on the first rot_dim dims with pairs (i, i +
    rot_dim / 2).  The step order and rotation convention are readings (the
    MSA pull request names the F32 projections, a gemma-style norm and 0.5
    partial rotary only).

    x [n_tok][d] f32; w_q, w_k [n_group * hd][d] f32; g_q, g_k [n_group][hd] f32.
    Returns (q [n_tok][n_group][hd], k [...]) in fp64 (None where not wanted)."""
    x = _c(x, np.float32)
    w_q, w_k = _c(w_q, np.float32), _c(w_k, np.float32)
    g_q, g_k = _c(g_q, np.float32), _c(g_k, np.float32)
    pos = _idx(pos)
    n_tok, d = x.shape
    hd = w_q.shape[0] // n_group
    if w_q.shape != (n_group * hd, d) or w_k.shape != w_q.shape or g_q.shape != (n_group, hd) or \
            g_k.shape != g_q.shape or pos.shape != (n_tok,):
        raise ValueError("index_project: inconsistent shapes")
    q = np.empty((n_tok, n_group, hd), np.float64) if want_q else None
    k = np.empty((n_tok, n_group, hd), np.float64) if want_k else None
    rc = lib().oracle_index_project(n_tok, d, n_group, hd, _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(g_q), _ptr(g_k),
                                    eps, theta, rot_dim, _ptr(pos), _ptr(q), _ptr(k))
    if rc != 0:
        raise ValueError("index_project: rot_dim must be even and at most the head dim")
    return q, k


KV_INT8, KV_Q4_0 = 1, 2


def kv_quantize(x_bits, fmt):
    """Quantize bf16 rows [..., L] (L a multiple of 32) per 32 values:
    symmetric absmax, int8 (fmt 1) or 4-bit (fmt 2, nibble-packed), one f32
    scale per 32 values (the quantizer rule is a reading; the pages give the
    format only).  Returns (codes uint8 [..., L] or [..., L / 2], scales f32
    [..., L / 32])."""
    x_bits = _c(x_bits, np.uint16)
    L = x_bits.shape[-1]
    n = x_bits.size // L
    codes = np.empty(x_bits.shape[:-1] + ((L if fmt == KV_INT8 else L // 2),), np.uint8)
    scales = np.empty(x_bits.shape[:-1] + (L // 32,), np.float32)
    if lib().oracle_kv_quantize(n, L, fmt, _ptr(x_bits), _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("kv_quantize: row length must be a multiple of 32, fmt 1 or 2")
    return codes, scales


def kv_dequantize(codes, scales, fmt):
    """codes * scale per element, fp64 [..., L]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    L = scales.shape[-1] * 32
    n = scales.size // (L // 32)
    out = np.empty(scales.shape[:-1] + (L,), np.float64)
    if lib().oracle_kv_dequantize(n, L, fmt, _ptr(codes), _ptr(scales), _ptr(out)) != 0:
        raise ValueError("kv_dequantize: bad format")
    return out


def sparse_attend_f64(k_cache, v_cache, stream, pos, q, sel, *, unit, scale, heads_per_group=16,
                      shared_across_groups=False):
    """sparse_attend over fp64 K/V caches [S][cap][G][D] (dequantized caches)."""
    k_cache = _c(k_cache, np.float64)
    v_cache = _c(v_cache, np.float64)
    q = _c(q, np.uint16)
    sel = _idx(sel)
    stream = _idx(stream)
    pos = _idx(pos)
    _, cap, G, D = k_cache.shape
    n_q = pos.size
    L = sel.shape[-1]
    q_stride, g_stride = (L, 0) if shared_across_groups else (G * L, L)
    out = np.empty((n_q, G * heads_per_group, D), np.float64)
    rc = lib().oracle_sparse_attend_f64(G, heads_per_group, D, float(scale), cap, _ptr(k_cache), _ptr(v_cache),
                                        n_q, _ptr(stream), _ptr(pos), _ptr(q), _ptr(sel), q_stride, g_stride,
                                        L, unit, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_sparse_attend_f64 failed: {rc}")
    return out
