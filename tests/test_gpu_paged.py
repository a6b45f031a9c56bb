"""GPU tests of paged caches (msa_cache.d_block_table): the same workload run
on per-stream caches and on page pools, with the logical blocks scattered
over the pool by a random permutation (spare pages left unused), must give
bit-identical appends, block scores, selections and attention outputs,
since paging changes only which rows are addressed.  The per-stream path is
itself checked against the fp64 oracle by the other GPU tests; one case here
also checks the paged path against the oracle directly.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W
from _gpu_common import DEV, check_attention, check_selection, dev, dev_bits, log

pytestmark = pytest.mark.gpu


def _table(n_stream, nb, seed, spare=3):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_stream * nb + spare).astype(np.int32)
    return perm[: n_stream * nb].reshape(n_stream, nb), n_stream * nb + spare


def _to_pool(x: torch.Tensor, table: np.ndarray, n_pages: int) -> torch.Tensor:
    """[S][cap][...] per-stream cache -> [n_pages * 128][...] pool."""
    S, cap = x.shape[:2]
    pool = torch.zeros((n_pages * 128,) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    for s in range(S):
        for b in range(table.shape[1]):
            lo, hi = 128 * b, min(128 * b + 128, cap)
            if lo >= hi:
                break
            pg = int(table[s, b])
            pool[128 * pg: 128 * pg + hi - lo] = x[s, lo:hi]
    return pool


def _msa_caches(wl, host, idx_f16=False, seed=1):
    S, cap = wl.n_stream, wl.cap
    nb = (cap + 127) // 128
    table, n_pages = _table(S, nb, seed)
    idx = torch.from_numpy(host["idx_k"].astype(np.float16) if idx_f16 else host["idx_k"]).to(DEV)
    k = dev_bits(host["k"], torch.bfloat16)
    v = dev_bits(host["v"], torch.bfloat16)
    flat = dict(idx=idx, k=k, v=v)
    paged = dict(idx=_to_pool(idx, table, n_pages), k=_to_pool(k, table, n_pages), v=_to_pool(v, table, n_pages),
                 table=dev(table))
    key = "idx_k_f16" if idx_f16 else "idx_k"
    c_flat = M.make_cache(k=k, v=v, **{key: idx})
    c_paged = M.make_cache(k=paged["k"], v=paged["v"], block_table=paged["table"], cap=cap, **{key: paged["idx"]})
    return flat, paged, c_flat, c_paged, table


def _ws(dims, op, n_q, max_pos):
    return torch.empty(max(M.workspace_bytes(dims, op, n_q, max_pos), 256), dtype=torch.uint8, device=DEV)


def _decode_both(wl, idx_f16=False, check_oracle=False):
    log(f"[paged decode] {wl.name}: streams={wl.n_stream} cap={wl.cap} n_q={wl.n_q} f16={idx_f16}")
    host, qs = W.caches(wl), W.queries(wl)
    flat, paged, c_flat, c_paged, table = _msa_caches(wl, host, idx_f16)
    dims = M.msa_dims(wl.top_k, W.SCALE)
    # append each query's own row into both layouts (cleared first)
    pairs = sorted(set(zip(wl.stream, wl.pos)))
    s_arr = np.array([a for a, _ in pairs], np.int32)
    p_arr = np.array([b for _, b in pairs], np.int32)
    si, pi = torch.from_numpy(s_arr).long(), torch.from_numpy(p_arr).long()
    prow = torch.from_numpy(table[s_arr, p_arr // 128].astype(np.int64) * 128 + p_arr % 128)
    for name in ("idx", "k", "v"):
        flat[name][si, pi] = 0
        paged[name][prow] = 0
    new = dict(idx_k_new=dev(host["idx_k"][s_arr, p_arr]), k_new=dev_bits(host["k"][s_arr, p_arr], torch.bfloat16),
               v_new=dev_bits(host["v"][s_arr, p_arr], torch.bfloat16))
    for c in (c_flat, c_paged):
        M.msa_index_append(dims, c, dev(s_arr), dev(p_arr), int(p_arr.max()), **new)
    torch.cuda.synchronize()
    for name in ("idx", "k", "v"):
        assert torch.equal(flat[name][si, pi], paged[name][prow]), f"paged append differs ({name})"
    n_q, nblk = wl.n_q, wl.max_pos // 128 + 1
    idx_q, stream, pos, q = dev(qs["idx_q"]), dev(qs["stream"]), dev(qs["pos"]), dev_bits(qs["q"], torch.bfloat16)
    res = []
    for c in (c_flat, c_paged):
        bs = torch.empty((n_q, 4, nblk), device=DEV)
        sel = torch.empty((n_q, 4, wl.top_k), dtype=torch.int32, device=DEV)
        n_sel = torch.empty((n_q, 4), dtype=torch.int32, device=DEV)
        out = torch.empty((n_q, 64, 128), device=DEV)
        M.msa_block_scores(dims, c, idx_q, stream, pos, wl.max_pos, bs)
        M.msa_select(dims, c, idx_q, stream, pos, wl.max_pos, sel, n_sel, _ws(dims, M.MSA_OP_SELECT, n_q, wl.max_pos))
        M.msa_attend_decode(dims, c, q, stream, pos, wl.max_pos, sel, out,
                            _ws(dims, M.MSA_OP_ATTEND_DECODE, n_q, wl.max_pos))
        res.append((bs, sel, n_sel, out))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b), "paged decode differs from per-stream"
    if check_oracle:
        keys = host["idx_k"].astype(np.float16).astype(np.float32) if idx_f16 else host["idx_k"]
        o_bs, o_sel, _ = oracle.msa_select(keys, qs["stream"], qs["pos"], qs["idx_q"], top_k=wl.top_k,
                                           nblk_out=nblk)
        equal, _ = check_selection(res[1][1].cpu().numpy(), o_sel, o_bs, qs["pos"], res[1][2].cpu().numpy())
        o_out = oracle.sparse_attend(host["k"], host["v"], qs["stream"], qs["pos"], qs["q"], o_sel, unit=128,
                                     scale=W.SCALE)
        wa, wr = check_attention(res[1][3].cpu().numpy(), o_out, mask_qg=equal)
        log(f"  paged vs oracle: {equal.sum()} of {equal.size} sets identical, attention max-abs {wa:.3e}")


def test_paged_decode_ragged_positions():
    pos = [0, 1, 127, 128, 129, 1000, 2047, 2048, 2049, 4095, 4999, 3333]
    _decode_both(W.Workload("paged", "msa_decode", 5, 5000, tuple(i % 5 for i in range(len(pos))), tuple(pos)),
                 check_oracle=True)


def test_paged_decode_fp16_index():
    pos = [0, 200, 4095, 4999, 2048]
    _decode_both(W.Workload("paged16", "msa_decode", 3, 5000, (0, 1, 2, 0, 1), tuple(pos)), idx_f16=True)


def test_paged_decode_top_k_64():
    _decode_both(W.Workload("paged64", "msa_decode", 2, 9000, (0, 1, 1), (8999, 5000, 8191), top_k=64))


def test_paged_prefill():
    wl = W.prefill_workload("paged_pf", 3000, 1900, 300, stream=1, n_stream=2)
    log(f"[paged prefill] {wl.name}")
    host, qs = W.caches(wl), W.queries(wl)
    flat, paged, c_flat, c_paged, table = _msa_caches(wl, host)
    dims = M.msa_dims(wl.top_k, W.SCALE)
    n_q, s0, pos0 = wl.n_q, wl.stream[0], wl.pos[0]
    idx_q, q = dev(qs["idx_q"]), dev_bits(qs["q"], torch.bfloat16)
    res = []
    for c in (c_flat, c_paged):
        sel = torch.empty((n_q, 4, wl.top_k), dtype=torch.int32, device=DEV)
        n_sel = torch.empty((n_q, 4), dtype=torch.int32, device=DEV)
        out = torch.empty((n_q, 64, 128), device=DEV)
        M.msa_select_prefill(dims, c, idx_q, s0, pos0, sel, n_sel,
                             _ws(dims, M.MSA_OP_SELECT_PREFILL, n_q, wl.max_pos))
        M.msa_attend_prefill(dims, c, q, s0, pos0, sel, out, _ws(dims, M.MSA_OP_ATTEND_PREFILL, n_q, wl.max_pos))
        res.append((sel, n_sel, out))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b), "paged prefill differs from per-stream"


def test_paged_dsa():
    wl = W.Workload("paged_dsa", "dsa_decode", 3, 5000, (0, 1, 2, 0), (4999, 3000, 127, 2100), top_k=2048)
    log(f"[paged dsa] {wl.name}")
    host, qs = W.caches(wl), W.queries(wl)
    S, cap = wl.n_stream, wl.cap
    nb = (cap + 127) // 128
    table, n_pages = _table(S, nb, 7)
    k = dev_bits(host["k"], torch.bfloat16)
    v = dev_bits(host["v"], torch.bfloat16)
    dsa_flat = torch.zeros((S, cap, 128), dtype=torch.float16, device=DEV)
    dsa_pool = torch.zeros((n_pages * 128, 128), dtype=torch.float16, device=DEV)
    c_flat = M.make_cache(k=k, v=v, dsa_k=dsa_flat)
    c_paged = M.make_cache(k=_to_pool(k, table, n_pages), v=_to_pool(v, table, n_pages), dsa_k=dsa_pool,
                           block_table=dev(table), cap=cap)
    dims = M.dsa_dims(wl.top_k, W.SCALE)
    st = torch.arange(S, dtype=torch.int32, device=DEV).repeat_interleave(cap)
    ps = torch.arange(cap, dtype=torch.int32, device=DEV).repeat(S)
    keys = dev_bits(host["dsa_k"].reshape(S * cap, -1), torch.float16)
    for c in (c_flat, c_paged):
        M.dsa_index_append(dims, c, st, ps, cap - 1, keys)
    torch.cuda.synchronize()
    assert torch.equal(_to_pool(dsa_flat, table, n_pages), dsa_pool), "paged DSA append differs"
    n_q = wl.n_q
    q_idx, stream, pos = dev_bits(qs["q_idx"], torch.float16), dev(qs["stream"]), dev(qs["pos"])
    q = dev_bits(qs["q"], torch.bfloat16)
    qh = W.queries_dsa_heads(wl, 32)
    q_h, w_h = dev_bits(qh["q_idx_h"], torch.float16), dev(qh["head_w"])
    res = []
    for c in (c_flat, c_paged):
        sel = torch.empty((n_q, wl.top_k), dtype=torch.int32, device=DEV)
        n_sel = torch.empty(n_q, dtype=torch.int32, device=DEV)
        out = torch.empty((n_q, 64, 128), device=DEV)
        M.dsa_select(dims, c, q_idx, stream, pos, wl.max_pos, sel, n_sel, _ws(dims, M.DSA_OP_SELECT, n_q, wl.max_pos))
        M.dsa_attend_decode(dims, c, q, stream, pos, wl.max_pos, sel, out,
                            _ws(dims, M.DSA_OP_ATTEND_DECODE, n_q, wl.max_pos))
        sel_h = torch.empty((n_q, wl.top_k), dtype=torch.int32, device=DEV)
        n_sel_h = torch.empty(n_q, dtype=torch.int32, device=DEV)
        M.dsa_select_heads(dims, c, q_h, w_h, stream, pos, wl.max_pos, sel_h, n_sel_h,
                           _ws(dims, M.DSA_OP_SELECT, n_q, wl.max_pos))
        res.append((sel, n_sel, out, sel_h, n_sel_h))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b), "paged DSA differs from per-stream"
