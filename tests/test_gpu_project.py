"""GPU parity of the indexer projection (msa_index_project) against the fp64
oracle, through the C ABI.

Tolerance (derived in tests/_tolerances.py, checked on the CPU in
tests/test_tolerance_models.py): a per-element bound from the f32 summation
model.  The error of an f32 sum of d_model products grows with the partial
sums it passes through, so with the output's own magnitude: sigma_y =
2^-24 / sqrt(3) * sqrt(d_model (y^2/3 + V/6)), V the sum of squared products.
The norm scales it by r (1 + gamma), the rotation mixes a pair; the bound is
10 sigma + 16 * 2^-24 |z| (the norm's and rotation's own roundings), e.g.
1.4e-5 for a typical output and 5.6e-5 for one of magnitude 5 at d_model
3072.  fp16 cache rows: within that bound plus one fp16 ulp of the exact
value (the f32 result rounded once).  Paged and per-stream caches:
bit-identical.  End to end: the selection made from the projected queries
and keys matches the oracle's selection on its own projected keys under the
near-tie rule.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W
from _gpu_common import DEV, check_selection, dev, log
from _tolerances import projection_bound

pytestmark = pytest.mark.gpu

def _proj(d_model, seed=0, rot_dim=W.PROJ_ROT_DIM):
    w = W.projection_weights(d_model, seed)
    t = {k: dev(v) for k, v in w.items()}
    pr = M.make_proj(w_q=t["w_q"], w_k=t["w_k"], g_q=t["g_q"], g_k=t["g_k"], eps=W.PROJ_EPS,
                     rope_theta=W.PROJ_THETA, rot_dim=rot_dim)
    return w, pr


def _run(d_model, stream, pos, n_stream, cap, *, f16=False, table=None, rot_dim=W.PROJ_ROT_DIM, seed=0):
    n_tok = len(pos)
    w, pr = _proj(d_model, seed, rot_dim)
    x = W.hidden_states(n_tok, d_model, seed)
    dims = M.msa_dims()
    if table is None:
        idx = torch.zeros((n_stream, cap, 4, 128), dtype=torch.float16 if f16 else torch.float32, device=DEV)
        kv = torch.zeros((n_stream, cap, 4, 128), dtype=torch.bfloat16, device=DEV)
        cache = M.make_cache(k=kv, v=kv, **{("idx_k_f16" if f16 else "idx_k"): idx})
    else:
        n_pages = int(table.max()) + 1
        idx = torch.zeros((n_pages * 128, 4, 128), dtype=torch.float32, device=DEV)
        kv = torch.zeros((n_pages * 128, 4, 128), dtype=torch.bfloat16, device=DEV)
        cache = M.make_cache(k=kv, v=kv, idx_k=idx, block_table=dev(table), cap=cap)
        p = np.asarray(pos)
        r = table[np.asarray(stream), p // 128].astype(np.int64) * 128 + p % 128
    idx_q = torch.empty((n_tok, 4, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_INDEX_PROJECT, n_tok, 0), 256), dtype=torch.uint8,
                     device=DEV)
    M.msa_index_project(dims, cache, pr, dev(x), dev(np.asarray(stream, np.int32)), dev(np.asarray(pos, np.int32)),
                        int(max(pos)), idx_q, ws)
    torch.cuda.synchronize()
    if table is None:
        rows = idx[torch.from_numpy(np.asarray(stream, np.int64)), torch.from_numpy(np.asarray(pos, np.int64))]
    else:
        rows = idx[torch.from_numpy(r)]
    oq, ok = oracle.index_project(x, w["w_q"], w["w_k"], w["g_q"], w["g_k"], np.asarray(pos, np.int32),
                                  eps=W.PROJ_EPS, theta=W.PROJ_THETA, rot_dim=rot_dim)
    bq = projection_bound(x, w["w_q"], w["g_q"], rot_dim, W.PROJ_EPS)
    bk = projection_bound(x, w["w_k"], w["g_k"], rot_dim, W.PROJ_EPS)
    return idx_q.cpu().numpy(), rows.float().cpu().numpy(), oq, ok, (idx, cache), (bq, bk)


def _check(gq, gk, oq, ok, bounds, f16=False):
    bq, bk = bounds
    rq = np.abs(gq - oq) / bq
    log(f"  q: max-abs {np.abs(gq - oq).max():.2e}, max error / bound {rq.max():.3f}")
    if f16:
        # the f32 value is within the bound of exact; one rounding to fp16 adds at most half an ulp
        ulp = np.spacing(np.abs(ok).astype(np.float16)).astype(np.float64)
        ek = ((np.abs(gk - ok) - bk) / ulp).max()
        log(f"  fp16 k: max (error - bound) = {ek:.2f} ulp")
        assert ek <= 1.0
    else:
        rk = np.abs(gk - ok) / bk
        log(f"  k: max-abs {np.abs(gk - ok).max():.2e}, max error / bound {rk.max():.3f}")
        assert rk.max() <= 1.0
    assert rq.max() <= 1.0


def test_project_small_ragged_tiles():
    rng = np.random.default_rng(1)
    pos = rng.choice(5000, size=70, replace=False).astype(np.int32)     # 2 token tiles, ragged
    stream = (np.arange(70) % 3).astype(np.int32)
    log("[project] 70 tokens, d_model 768, f32 cache")
    gq, gk, oq, ok, _, bnd = _run(768, stream, pos, 3, 5000)
    _check(gq, gk, oq, ok, bnd)


def test_project_minimal_d_model_no_rotation():
    log("[project] 5 tokens, d_model 32, rot_dim 0")
    gq, gk, oq, ok, _, bnd = _run(32, [0, 0, 1, 1, 0], [0, 1, 2, 3, 4000], 2, 4096, rot_dim=0)
    _check(gq, gk, oq, ok, bnd)


def test_project_fp16_index_cache():
    rng = np.random.default_rng(2)
    pos = rng.choice(3000, size=40, replace=False).astype(np.int32)
    log("[project] 40 tokens, d_model 768, fp16 cache")
    gq, gk, oq, ok, _, bnd = _run(768, np.zeros(40, np.int32), pos, 1, 3000, f16=True)
    _check(gq, gk, oq, ok, bnd, f16=True)


def test_project_paged_equals_per_stream():
    rng = np.random.default_rng(3)
    pos = rng.choice(5000, size=50, replace=False).astype(np.int32)
    stream = (np.arange(50) % 2).astype(np.int32)
    table = rng.permutation(2 * 40 + 5)[:80].astype(np.int32).reshape(2, 40)
    log("[project] paged vs per-stream")
    a = _run(768, stream, pos, 2, 5000)
    b = _run(768, stream, pos, 2, 5000, table=table)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_project_decode_32_tokens_d3072():
    """Decode shape: one token per stream at position 32767 (32 streams); the
    hidden size is split 32 ways."""
    S, cap = 32, 32768
    log("[project] decode 32 tokens, d_model 3072")
    gq, gk, oq, ok, _, bnd = _run(W.PROJ_D_MODEL, np.arange(S, dtype=np.int32), np.full(S, cap - 1, np.int32), S, cap)
    _check(gq, gk, oq, ok, bnd)


def test_project_then_select_4x4096():
    """Hidden states -> projection (every key of 4 streams x 4096 positions)
    -> block selection of the last position of each stream, against the
    oracle's selection on the oracle's own projected keys."""
    S, cap, d = 4, 4096, 768
    log("[project] 4 x 4096 keys, d_model 768, then block selection")
    stream = np.repeat(np.arange(S, dtype=np.int32), cap)
    pos = np.tile(np.arange(cap, dtype=np.int32), S)
    gq, gk, oq, ok, (idx, cache), bnd = _run(d, stream, pos, S, cap)
    _check(gq, gk, oq, ok, bnd)
    last = np.arange(S) * cap + cap - 1
    keys = ok.reshape(S, cap, 4, 128).astype(np.float32)
    dims = M.msa_dims()
    st_d, pos_d = dev(np.arange(S, dtype=np.int32)), dev(np.full(S, cap - 1, np.int32))
    sel = torch.empty((S, 4, 16), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((S, 4), dtype=torch.int32, device=DEV)
    ws = torch.empty(M.workspace_bytes(dims, M.MSA_OP_SELECT, S, cap - 1), dtype=torch.uint8, device=DEV)
    M.msa_select(dims, cache, torch.from_numpy(gq[last]).to(DEV), st_d, pos_d, cap - 1, sel, n_sel, ws)
    torch.cuda.synchronize()
    o_bs, o_sel, _ = oracle.msa_select(keys, np.arange(S, dtype=np.int32), np.full(S, cap - 1, np.int32),
                                       oq[last].astype(np.float32))
    equal, n_diff = check_selection(sel.cpu().numpy(), o_sel, o_bs, np.full(S, cap - 1), n_sel.cpu().numpy())
    log(f"  selection from projected inputs: {equal.sum()} of {equal.size} sets identical, {n_diff} near-tie swaps")


def test_project_prefill_4096_d3072():
    log("[project] prefill 4096 tokens at 28672, d_model 3072")
    pos = np.arange(28672, 32768, dtype=np.int32)
    gq, gk, oq, ok, _, bnd = _run(W.PROJ_D_MODEL, np.zeros(4096, np.int32), pos, 1, 32768)
    _check(gq, gk, oq, ok, bnd)
