"""Seeded synthetic workloads for the MSA / DSA hot path.

This module holds the input recipe and the workload registry only; it contains
none of the method's arithmetic (no scores, pooling, selection or attention).
Both the oracle-side tests and the HIP-side tests and benchmark draw their
inputs from here, and from nowhere else.

Recipe (stated once, used everywhere):
  * Head geometry of the MiniMax-M3 sparse layer described in the MSA pull
    request ("Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support",
    Overview and review thread): 4 GQA groups, 16 query heads per group
    (64 query heads, 4 KV heads), head_dim 128, one 128-dim indexer head per
    group, block 128, top-16.
  * Caches are per stream and token-major: idx_k [cap][G][128] f32,
    K and V [cap][G][128] bf16; slot == position.
  * Every tensor is drawn with numpy's PCG64 generator seeded by
    SeedSequence([seed, tag, index]) where `tag` names the tensor kind and
    `index` is the stream (caches) or the query (query tensors); so any single
    stream or query can be regenerated on its own, bit for bit.
  * Gaussian values are drawn as float32 N(0, 1) and rounded once to the
    storage type (bf16 or fp16, round-to-nearest-even via torch's casts).
  * Integer indexer workloads draw integers uniformly from -8..8 inclusive and
    store them as f32 (all partial sums are exact in f32).
  * The prefill workload multiplies the f32 indexer vectors by
    float32(1/sqrt(128)) after drawing.
  * Indexer projection: hidden states float32 N(0, 1) [n_tok][d_model];
    F32 projection weights N(0, 1) * float32(1/sqrt(d_model)), [512][d_model]
    each for queries and keys (4 groups x 128); norm gains float32
    0.1 * N(0, 1) [4][128] each; eps 1e-6, RoPE base 10000 on 64 of 128 dims.
    d_model defaults to 3072 (the pages give no hidden size for the full
    model; the pull request's random-weight test model uses 768).
  * Multi-head DSA indexer (n_ihead = 32 heads, the GLM geometry the DSA pull
    request reports): per query, n_ihead fp16 query rows drawn as above and
    n_ihead f32 head weights drawn as float32 N(0, 1) times
    float32(1/sqrt(n_ihead)) (both signs occur).
There is no dataset: the pages measure on wikitext-2 with real weights, which
these synthetic tensors of the real geometry stand in for.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

N_GROUP = 4
HEADS_PER_GROUP = 16
HEAD_DIM = 128
IDX_DIM = 128
BLOCK = 128
TOP_K = 16
DSA_TOP_K = 2048
SCALE = float(np.float32(1.0 / math.sqrt(HEAD_DIM)))   # the f32 value both sides use

# tensor-kind tags of the seed sequence
_T_IDX_K, _T_K, _T_V, _T_IDX_Q, _T_Q, _T_DSA_K, _T_DSA_Q = 1, 2, 3, 4, 5, 6, 7
_T_DSA_QH, _T_DSA_W = 8, 9
_T_X, _T_WQ, _T_WK, _T_GQ, _T_GK = 10, 11, 12, 13, 14
PROJ_D_MODEL = 3072
PROJ_EPS = 1e-6
PROJ_THETA = 10000.0
PROJ_ROT_DIM = 64
DSA_N_IHEAD = 32


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "msa_decode" | "msa_prefill" | "dsa_decode"
    n_stream: int
    cap: int                  # slots per stream
    stream: Tuple[int, ...]   # per query
    pos: Tuple[int, ...]      # per query
    idx_dist: str = "normal"  # "int8" | "normal" | "normal_scaled"
    seed: int = 0
    block: int = BLOCK
    top_k: int = TOP_K

    @property
    def n_q(self) -> int:
        return len(self.pos)

    @property
    def max_pos(self) -> int:
        return max(self.pos)


def decode_workload(name, n_stream, ctx, idx_dist="normal", seed=0, kind="msa_decode",
                    top_k=None, cap=None):
    """One query per stream at position ctx - 1 (the cache holds ctx tokens)."""
    cap = ctx if cap is None else cap
    if top_k is None:
        top_k = DSA_TOP_K if kind == "dsa_decode" else TOP_K
    return Workload(name, kind, n_stream, cap, tuple(range(n_stream)),
                    tuple([ctx - 1] * n_stream), idx_dist, seed, BLOCK, top_k)


def prefill_workload(name, ctx, pos0, n_q, idx_dist="normal_scaled", seed=0, stream=0,
                     n_stream=1):
    return Workload(name, "msa_prefill", n_stream, ctx, tuple([stream] * n_q),
                    tuple(range(pos0, pos0 + n_q)), idx_dist, seed, BLOCK, TOP_K)


# The five measured configurations.
CONFIGS: Dict[str, Workload] = {
    "decode_1x4k_int": decode_workload("decode_1x4k_int", 1, 4096, "int8"),
    "decode_32x32k": decode_workload("decode_32x32k", 32, 32768),
    "decode_8x128k": decode_workload("decode_8x128k", 8, 131072),
    "prefill_4096_at_32k": prefill_workload("prefill_4096_at_32k", 32768, 28672, 4096),
    "dsa_16x64k": decode_workload("dsa_16x64k", 16, 65536, kind="dsa_decode"),
}


def _rng(seed: int, tag: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


def _normal_f32(rng, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> fp16 bit patterns (uint16), round-to-nearest-even."""
    return np.ascontiguousarray(x, np.float32).astype(np.float16).view(np.uint16)


def _indexer_values(wl: Workload, rng, shape) -> np.ndarray:
    if wl.idx_dist == "int8":
        return rng.integers(-8, 9, size=shape, dtype=np.int8).astype(np.float32)
    x = _normal_f32(rng, shape)
    if wl.idx_dist == "normal_scaled":
        x *= np.float32(1.0 / math.sqrt(IDX_DIM))
    elif wl.idx_dist != "normal":
        raise ValueError(wl.idx_dist)
    return x


# ---------------------------------------------------------------------------
# Per-stream cache contents and per-query tensors
# ---------------------------------------------------------------------------
def stream_idx_k(wl: Workload, s: int) -> np.ndarray:
    """[cap][G][IDX_DIM] f32 index keys of stream s (MSA)."""
    return _indexer_values(wl, _rng(wl.seed, _T_IDX_K, s), (wl.cap, N_GROUP, IDX_DIM))


def stream_kv(wl: Workload, s: int) -> Tuple[np.ndarray, np.ndarray]:
    """K and V [cap][G][HEAD_DIM] bf16 bits of stream s."""
    k = to_bf16_bits(_normal_f32(_rng(wl.seed, _T_K, s), (wl.cap, N_GROUP, HEAD_DIM)))
    v = to_bf16_bits(_normal_f32(_rng(wl.seed, _T_V, s), (wl.cap, N_GROUP, HEAD_DIM)))
    return k, v


def stream_dsa_keys(wl: Workload, s: int) -> np.ndarray:
    """[cap][IDX_DIM] raw (un-rotated) fp16 indexer keys of stream s (DSA)."""
    return to_f16_bits(_normal_f32(_rng(wl.seed, _T_DSA_K, s), (wl.cap, IDX_DIM)))


def query_idx(wl: Workload, i: int) -> np.ndarray:
    """[G][IDX_DIM] f32 indexer query of query i (MSA)."""
    return _indexer_values(wl, _rng(wl.seed, _T_IDX_Q, i), (N_GROUP, IDX_DIM))


def query_q(wl: Workload, i: int) -> np.ndarray:
    """[G*HEADS_PER_GROUP][HEAD_DIM] bf16 bits of query i."""
    return to_bf16_bits(_normal_f32(_rng(wl.seed, _T_Q, i), (N_GROUP * HEADS_PER_GROUP, HEAD_DIM)))


def query_dsa(wl: Workload, i: int) -> np.ndarray:
    """[IDX_DIM] fp16 bits of the DSA indexer query of query i."""
    return to_f16_bits(_normal_f32(_rng(wl.seed, _T_DSA_Q, i), (IDX_DIM,)))


def query_dsa_heads(wl: Workload, i: int, n_head: int = DSA_N_IHEAD) -> np.ndarray:
    """[n_head][IDX_DIM] fp16 bits of the multi-head DSA indexer query of query i."""
    return to_f16_bits(_normal_f32(_rng(wl.seed, _T_DSA_QH, i), (n_head, IDX_DIM)))


def head_weights(wl: Workload, i: int, n_head: int = DSA_N_IHEAD) -> np.ndarray:
    """[n_head] f32 indexer head weights of query i."""
    return _normal_f32(_rng(wl.seed, _T_DSA_W, i), (n_head,)) * np.float32(1.0 / math.sqrt(n_head))


def queries_dsa_heads(wl: Workload, n_head: int = DSA_N_IHEAD,
                      idx: Optional[List[int]] = None) -> Dict[str, np.ndarray]:
    """Stacked multi-head indexer queries: q_idx_h [n_q][n_head][IDX_DIM] fp16
    bits and head_w [n_q][n_head] f32."""
    idx = list(range(wl.n_q)) if idx is None else list(idx)
    if not idx:
        return {"q_idx_h": np.zeros((0, n_head, IDX_DIM), np.uint16), "head_w": np.zeros((0, n_head), np.float32)}
    return {"q_idx_h": np.stack([query_dsa_heads(wl, i, n_head) for i in idx]),
            "head_w": np.stack([head_weights(wl, i, n_head) for i in idx]).astype(np.float32)}


def queries(wl: Workload, idx: Optional[List[int]] = None) -> Dict[str, np.ndarray]:
    """Stacked query tensors of the given query indices (all by default)."""
    idx = list(range(wl.n_q)) if idx is None else list(idx)
    out = {
        "stream": np.array([wl.stream[i] for i in idx], np.int32),
        "pos": np.array([wl.pos[i] for i in idx], np.int32),
        "q": np.stack([query_q(wl, i) for i in idx]) if idx else
             np.zeros((0, N_GROUP * HEADS_PER_GROUP, HEAD_DIM), np.uint16),
    }
    if wl.kind == "dsa_decode":
        out["q_idx"] = (np.stack([query_dsa(wl, i) for i in idx]) if idx
                        else np.zeros((0, IDX_DIM), np.uint16))
    else:
        out["idx_q"] = (np.stack([query_idx(wl, i) for i in idx]) if idx
                        else np.zeros((0, N_GROUP, IDX_DIM), np.float32))
    return out


def caches(wl: Workload, streams: Optional[List[int]] = None) -> Dict[str, np.ndarray]:
    """Host cache arrays of the given streams, stacked [len(streams)][cap][...].

    Slots past a stream's largest query position are left as drawn (they are
    never visible to any query of the workload)."""
    streams = list(range(wl.n_stream)) if streams is None else list(streams)
    n = len(streams)
    out: Dict[str, np.ndarray] = {}
    if wl.kind == "dsa_decode":
        out["dsa_k"] = np.empty((n, wl.cap, IDX_DIM), np.uint16)
    else:
        out["idx_k"] = np.empty((n, wl.cap, N_GROUP, IDX_DIM), np.float32)
    out["k"] = np.empty((n, wl.cap, N_GROUP, HEAD_DIM), np.uint16)
    out["v"] = np.empty((n, wl.cap, N_GROUP, HEAD_DIM), np.uint16)
    for j, s in enumerate(streams):
        if wl.kind == "dsa_decode":
            out["dsa_k"][j] = stream_dsa_keys(wl, s)
        else:
            out["idx_k"][j] = stream_idx_k(wl, s)
        out["k"][j], out["v"][j] = stream_kv(wl, s)
    return out


def hidden_states(n_tok: int, d_model: int = PROJ_D_MODEL, seed: int = 0) -> np.ndarray:
    """[n_tok][d_model] f32 hidden states entering the indexer projection."""
    return _normal_f32(_rng(seed, _T_X, 0), (n_tok, d_model))


def projection_weights(d_model: int = PROJ_D_MODEL, seed: int = 0) -> Dict[str, np.ndarray]:
    """F32 indexer projection weights w_q, w_k [512][d_model] and norm gains
    g_q, g_k [4][128]."""
    scale = np.float32(1.0 / math.sqrt(d_model))
    return {
        "w_q": _normal_f32(_rng(seed, _T_WQ, 0), (N_GROUP * IDX_DIM, d_model)) * scale,
        "w_k": _normal_f32(_rng(seed, _T_WK, 0), (N_GROUP * IDX_DIM, d_model)) * scale,
        "g_q": _normal_f32(_rng(seed, _T_GQ, 0), (N_GROUP, IDX_DIM)) * np.float32(0.1),
        "g_k": _normal_f32(_rng(seed, _T_GK, 0), (N_GROUP, IDX_DIM)) * np.float32(0.1),
    }
