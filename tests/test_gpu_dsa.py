"""GPU parity of the DSA lightning-indexer variant (Hadamard key rotation into
the fp16 cache, token top-k selection, attention over the kept tokens)
against the fp64 oracle, through the C ABI.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W
from _gpu_common import DEV, GpuWorkload, check_attention, check_token_selection, dev, dev_bits, host_bits, log

pytestmark = pytest.mark.gpu


def _dsa_parity(wl: W.Workload, host=None):
    log(f"[dsa] {wl.name}: streams={wl.n_stream} cap={wl.cap} n_q={wl.n_q} top_k={wl.top_k}")
    dims = M.dsa_dims(wl.top_k, W.SCALE)
    gw = GpuWorkload(wl, host)
    gw.append_own_rows()             # rotates every key into the fp16 cache
    torch.cuda.synchronize()
    # rotation parity: bit-exact (exact fp64 transform, one RNE rounding)
    o_rot = oracle.dsa_rotate(gw.host["dsa_k"])
    g_rot = host_bits(gw.dsa_k)
    n_bad = int((g_rot != o_rot).sum())
    assert n_bad == 0, f"{n_bad} rotated key elements differ"
    q_idx = dev_bits(gw.qs["q_idx"], torch.float16)
    sel = torch.empty((wl.n_q, wl.top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty(wl.n_q, dtype=torch.int32, device=DEV)
    M.dsa_select(dims, gw.cache, q_idx, gw.stream, gw.pos, wl.max_pos, sel, n_sel,
                 gw.ws(dims, M.DSA_OP_SELECT))
    torch.cuda.synchronize()
    o_sel, o_nsel, scores = oracle.dsa_select(o_rot, gw.qs["stream"], gw.qs["pos"], gw.qs["q_idx"],
                                              top_k=wl.top_k, want_scores=True)
    equal = check_token_selection(sel.cpu().numpy(), n_sel.cpu().numpy(), o_sel, o_nsel, scores,
                                   gw.qs["pos"], wl.top_k)
    log(f"  selection: {equal.sum()} of {len(equal)} queries identical")
    o_out = oracle.sparse_attend(gw.host["k"], gw.host["v"], gw.qs["stream"], gw.qs["pos"], gw.qs["q"],
                                 o_sel, unit=1, scale=W.SCALE, shared_across_groups=True)

    def attend(sel_dev):
        out = torch.empty((wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
        M.dsa_attend_decode(dims, gw.cache, gw.q, gw.stream, gw.pos, wl.max_pos, sel_dev, out,
                            gw.ws(dims, M.DSA_OP_ATTEND_DECODE))
        return out.cpu().numpy()

    out_o = attend(dev(o_sel))
    wa, wr = check_attention(out_o, o_out)
    log(f"  attention on the oracle selection: max-abs {wa:.3e}, rel-L2 {wr:.3e}")
    check_attention(attend(sel), o_out, mask_qg=np.repeat(equal[:, None], 4, 1))
    # msa_attend_decode with block 1 is the same call
    out_m = torch.empty((wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
    M.msa_attend_decode(dims, gw.cache, gw.q, gw.stream, gw.pos, wl.max_pos, dev(o_sel), out_m,
                        gw.ws(dims, M.MSA_OP_ATTEND_DECODE))
    assert np.array_equal(out_m.cpu().numpy(), out_o)


def test_dsa_small_ragged():
    # ragged cap; positions below and above top_k; a short context (p + 1 <= top_k)
    wl = W.Workload("dsa_small", "dsa_decode", 3, 3000, (0, 1, 2, 0, 1), (2999, 63, 1500, 64, 0),
                    top_k=64)
    _dsa_parity(wl)


def test_dsa_dense_when_context_fits():
    wl = W.Workload("dsa_dense", "dsa_decode", 2, 2048, (0, 1), (2047, 1000), top_k=2048)
    _dsa_parity(wl)


def test_dsa_all_scores_tied():
    # every key identical: all scores tie, the lowest ids win; the boundary
    # bin holds every key, more than the candidate list keeps in LDS
    wl = W.Workload("dsa_ties", "dsa_decode", 1, 6000, (0, 0), (5999, 4500), top_k=100)
    host = W.caches(wl)
    host["dsa_k"][:] = host["dsa_k"][0, 0]
    _dsa_parity(wl, host)


def test_dsa_full_16x64k():
    _dsa_parity(W.CONFIGS["dsa_16x64k"])


def test_dsa_topk_context_over_64k_exact():
    """Contexts above 65536 keys take the streaming top-k (the register one
    holds at most 65536 keys per query): integer scores, ties everywhere,
    bit-exact against the oracle, one query below and one above 65536."""
    S, cap, top_k = 1, 70000, 2048
    rng = np.random.default_rng(23)
    k_rot = rng.integers(-2, 3, size=(S, cap, 128)).astype(np.float16)
    pos = np.array([69999, 40000], np.int32)
    stream = np.array([0, 0], np.int32)
    q = rng.integers(-1, 2, size=(2, 128)).astype(np.float16)
    log("[dsa] exact ties, context 70000")
    dims = M.dsa_dims(top_k, W.SCALE)
    cache = M.make_cache(k=torch.zeros((S, cap, 4, 128), dtype=torch.bfloat16, device=DEV),
                         v=torch.zeros((S, cap, 4, 128), dtype=torch.bfloat16, device=DEV),
                         dsa_k=torch.from_numpy(k_rot).to(DEV))
    sel = torch.empty((2, top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty(2, dtype=torch.int32, device=DEV)
    ws = torch.empty(M.workspace_bytes(dims, M.DSA_OP_SELECT, 2, int(pos.max())), dtype=torch.uint8, device=DEV)
    M.dsa_select(dims, cache, torch.from_numpy(q).to(DEV), dev(stream), dev(pos), int(pos.max()), sel, n_sel, ws)
    torch.cuda.synchronize()
    o_sel, o_nsel, _ = oracle.dsa_select(k_rot.view(np.uint16), stream, pos, q.view(np.uint16), top_k=top_k)
    assert np.array_equal(n_sel.cpu().numpy(), o_nsel)
    assert np.array_equal(sel.cpu().numpy(), o_sel), "selection differs from the oracle"


@pytest.mark.parametrize("top_k", [2048, 64])
def test_dsa_topk_with_ties_exact(top_k):
    """Integer keys and queries make every score an exact small integer, so
    ties are everywhere (far more keys share the boundary score than the LDS
    candidate list holds) and the selection must equal the oracle's bit for
    bit (ties to the lower token id), including a query shorter than top_k."""
    S, cap = 2, 40000
    rng = np.random.default_rng(17)
    k_rot = rng.integers(-2, 3, size=(S, cap, 128)).astype(np.float16)
    pos = np.array([39999, 1500, 20000, 17000], np.int32)
    stream = np.array([0, 1, 1, 0], np.int32)
    q = rng.integers(-1, 2, size=(4, 128)).astype(np.float16)
    log(f"[dsa] exact ties, top_k {top_k}")
    dims = M.dsa_dims(top_k, W.SCALE)
    dsa_k = torch.from_numpy(k_rot).to(DEV)
    kv = torch.zeros((S, cap, 4, 128), dtype=torch.bfloat16, device=DEV)
    cache = M.make_cache(k=kv, v=kv, dsa_k=dsa_k)
    sel = torch.empty((4, top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty(4, dtype=torch.int32, device=DEV)
    ws = torch.empty(M.workspace_bytes(dims, M.DSA_OP_SELECT, 4, int(pos.max())), dtype=torch.uint8, device=DEV)
    M.dsa_select(dims, cache, torch.from_numpy(q).to(DEV), dev(stream), dev(pos), int(pos.max()), sel, n_sel, ws)
    torch.cuda.synchronize()
    o_sel, o_nsel, _ = oracle.dsa_select(k_rot.view(np.uint16), stream, pos, q.view(np.uint16), top_k=top_k)
    assert np.array_equal(n_sel.cpu().numpy(), o_nsel)
    assert np.array_equal(sel.cpu().numpy(), o_sel), "selection differs from the oracle"


@pytest.mark.parametrize("ints", [True, False])
def test_dsa_topk_chunked_equals_one_workgroup(ints):
    """Calls of at most 32 queries over more than 8192 keys rank each query's
    scores over one workgroup per 8192-key chunk; larger calls use one
    workgroup per query.  Both are exact, so 40 queries in one call and their
    first 8 and last 32 in calls of their own select the same ids bit for
    bit (integer scores: ties everywhere, also equal to the oracle's; Gaussian
    keys: distinct scores), at context lengths across chunk edges."""
    S, cap, top_k = 2, 30000, 2048
    rng = np.random.default_rng(29 if ints else 31)
    if ints:
        k_rot = rng.integers(-2, 3, size=(S, cap, 128)).astype(np.float16)
        q = rng.integers(-1, 2, size=(40, 128)).astype(np.float16)
    else:
        k_rot = rng.standard_normal((S, cap, 128)).astype(np.float16)
        q = rng.standard_normal((40, 128)).astype(np.float16)
    pos = rng.integers(2048, cap, size=40).astype(np.int32)
    pos[:6] = [8191, 8192, 16383, 16384, 29999, 2047]
    stream = rng.integers(0, S, size=40).astype(np.int32)
    log(f"[dsa] chunked vs one-workgroup top-k, integer scores {ints}")
    dims = M.dsa_dims(top_k, W.SCALE)
    kv = torch.zeros((S, cap, 4, 128), dtype=torch.bfloat16, device=DEV)
    cache = M.make_cache(k=kv, v=kv, dsa_k=torch.from_numpy(k_rot).to(DEV))
    qd = torch.from_numpy(q).to(DEV)

    def select(lo, hi):
        n = hi - lo
        sel = torch.empty((n, top_k), dtype=torch.int32, device=DEV)
        n_sel = torch.empty(n, dtype=torch.int32, device=DEV)
        mp = int(pos[lo:hi].max())
        ws = torch.empty(M.workspace_bytes(dims, M.DSA_OP_SELECT, n, mp), dtype=torch.uint8, device=DEV)
        M.dsa_select(dims, cache, qd[lo:hi].contiguous(), dev(stream[lo:hi]), dev(pos[lo:hi]), mp, sel, n_sel, ws)
        torch.cuda.synchronize()
        return sel.cpu().numpy(), n_sel.cpu().numpy()

    s_all, n_all = select(0, 40)
    s_a, n_a = select(0, 8)
    s_b, n_b = select(8, 40)
    assert np.array_equal(np.concatenate([s_a, s_b]), s_all)
    assert np.array_equal(np.concatenate([n_a, n_b]), n_all)
    if ints:
        o_sel, o_nsel, _ = oracle.dsa_select(k_rot.view(np.uint16), stream, pos, q.view(np.uint16), top_k=top_k)
        assert np.array_equal(n_all, o_nsel)
        assert np.array_equal(s_all, o_sel), "selection differs from the oracle"


def test_dsa_topk_boundary_tie_list_over_2048():
    """5000 keys share the boundary score (a planted mid-level key), 1500 rank
    above it: the chunked top-k's boundary list holds about 5000 entries,
    more than it loads ahead of its counts but fewer than its LDS copy
    holds, and the kept ties are the lowest ids.  Exact against the oracle."""
    S, cap, top_k = 1, 30000, 2048
    rng = np.random.default_rng(37)
    k_rot = rng.integers(-1, 2, size=(S, cap, 128)).astype(np.float16)
    ids = rng.permutation(cap)
    k_rot[0, ids[:1500]] = 1.0                                   # score 128
    k_rot[0, ids[1500:6500]] = np.where(np.arange(128) < 64, 1.0, 0.0).astype(np.float16)   # score 64
    q = np.ones((2, 128), np.float16)
    pos = np.array([29999, 21000], np.int32)
    stream = np.zeros(2, np.int32)
    log("[dsa] boundary tie list over 2048 entries")
    dims = M.dsa_dims(top_k, W.SCALE)
    kv = torch.zeros((S, cap, 4, 128), dtype=torch.bfloat16, device=DEV)
    cache = M.make_cache(k=kv, v=kv, dsa_k=torch.from_numpy(k_rot).to(DEV))
    sel = torch.empty((2, top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty(2, dtype=torch.int32, device=DEV)
    ws = torch.empty(M.workspace_bytes(dims, M.DSA_OP_SELECT, 2, int(pos.max())), dtype=torch.uint8, device=DEV)
    M.dsa_select(dims, cache, torch.from_numpy(q).to(DEV), dev(stream), dev(pos), int(pos.max()), sel, n_sel, ws)
    torch.cuda.synchronize()
    o_sel, o_nsel, _ = oracle.dsa_select(k_rot.view(np.uint16), stream, pos, q.view(np.uint16), top_k=top_k)
    assert np.array_equal(n_sel.cpu().numpy(), o_nsel)
    assert np.array_equal(sel.cpu().numpy(), o_sel), "selection differs from the oracle"


@pytest.mark.parametrize("n_stream,ctx", [(4, 20000), (3, 3000)])
def test_dsa_step_graph_replay_matches_eager(n_stream, ctx):
    """The DSA decode step (append, select, attend) captured into a HIP graph
    and replayed six times, with eager work and synchronisations in between
    (outputs cleared, both workspaces cleared before one replay, an eager
    step before another), reproduces the eager step bit for bit every time:
    the chunked top-k (4 queries over 20000 keys) and the one-workgroup
    register top-k (3 queries over 3000)."""
    wl = W.Workload(f"dsa_graph_{ctx}", "dsa_decode", n_stream, ctx, tuple(range(n_stream)),
                    tuple(ctx - 1 - 7 * j for j in range(n_stream)), top_k=2048)
    log(f"[dsa] graph replay: {wl.n_q} queries over {ctx} slots")
    gw = GpuWorkload(wl)
    gw.append_own_rows()
    dims = M.dsa_dims(wl.top_k, W.SCALE)
    st, ps = gw.qs["stream"].astype(np.int64), gw.qs["pos"].astype(np.int64)
    new_key = dev_bits(gw.host["dsa_k"][st, ps], torch.float16)
    new_k = dev_bits(gw.host["k"][st, ps], torch.bfloat16)
    new_v = dev_bits(gw.host["v"][st, ps], torch.bfloat16)
    q_idx = dev_bits(gw.qs["q_idx"], torch.float16)
    sel = torch.empty((wl.n_q, wl.top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty(wl.n_q, dtype=torch.int32, device=DEV)
    out = torch.empty((wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
    ws_sel = gw.ws(dims, M.DSA_OP_SELECT)
    ws_att = gw.ws(dims, M.DSA_OP_ATTEND_DECODE)

    def step():
        M.dsa_index_append(dims, gw.cache, gw.stream, gw.pos, wl.max_pos, new_key, new_k, new_v)
        M.dsa_select(dims, gw.cache, q_idx, gw.stream, gw.pos, wl.max_pos, sel, n_sel, ws_sel)
        M.dsa_attend_decode(dims, gw.cache, gw.q, gw.stream, gw.pos, wl.max_pos, sel, out, ws_att)

    step()
    torch.cuda.synchronize()
    ref_out, ref_sel, ref_n = out.clone(), sel.clone(), n_sel.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(6):
        out.zero_()
        sel.fill_(-7)
        n_sel.fill_(-7)
        if r == 1:
            ws_sel.zero_()
            ws_att.zero_()
        elif r == 3:
            step()
            out.zero_()
            sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: output differs"
        assert torch.equal(sel, ref_sel) and torch.equal(n_sel, ref_n), f"replay {r}: selection differs"
