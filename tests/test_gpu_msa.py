"""GPU parity of the MSA hot path (append, block scores, top-16 selection,
decode and prefill sparse attention) against the fp64 oracle, through the
C ABI.  Sizes: small ragged cases that span several tiles, plus the five
measured workloads at full size, every query compared.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W
from _gpu_common import (DEV, GpuWorkload, check_attention, check_selection, dev, dev_bits, host_bits, log)

pytestmark = pytest.mark.gpu


def _select_gpu(gw: GpuWorkload, dims):
    n_q = gw.wl.n_q
    sel = torch.empty((n_q, 4, dims.top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((n_q, 4), dtype=torch.int32, device=DEV)
    M.msa_select(dims, gw.cache, dev(gw.qs["idx_q"]), gw.stream, gw.pos, gw.max_pos, sel, n_sel,
                 gw.ws(dims, M.MSA_OP_SELECT))
    return sel, n_sel


def _attend_gpu(gw: GpuWorkload, dims, sel_dev):
    out = torch.empty((gw.wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
    M.msa_attend_decode(dims, gw.cache, gw.q, gw.stream, gw.pos, gw.max_pos, sel_dev, out,
                        gw.ws(dims, M.MSA_OP_ATTEND_DECODE))
    return out


def _decode_parity(wl: W.Workload, exact: bool = False, host=None):
    log(f"[msa decode] {wl.name}: streams={wl.n_stream} cap={wl.cap} n_q={wl.n_q} top_k={wl.top_k}")
    dims = M.msa_dims(wl.top_k, W.SCALE)
    gw = GpuWorkload(wl, host)
    gw.append_own_rows()
    # append parity: the written rows are the host rows, bit for bit
    for s, p in zip(wl.stream[:4], wl.pos[:4]):
        assert np.array_equal(gw.idx_k[s, p].cpu().numpy(), gw.host["idx_k"][s, p])
        assert np.array_equal(host_bits(gw.k[s, p]), gw.host["k"][s, p])
        assert np.array_equal(host_bits(gw.v[s, p]), gw.host["v"][s, p])
    # block scores
    nblk = wl.max_pos // 128 + 1
    bs = torch.empty((wl.n_q, 4, nblk), dtype=torch.float32, device=DEV)
    M.msa_block_scores(dims, gw.cache, dev(gw.qs["idx_q"]), gw.stream, gw.pos, wl.max_pos, bs)
    sel, n_sel = _select_gpu(gw, dims)
    torch.cuda.synchronize()
    o_bs, o_sel, o_nsel = oracle.msa_select(gw.host["idx_k"], gw.qs["stream"], gw.qs["pos"],
                                            gw.qs["idx_q"], top_k=wl.top_k, nblk_out=nblk)
    g_bs = bs.cpu().numpy()
    if exact:
        assert np.array_equal(g_bs.astype(np.float64), o_bs), "block scores not bit-exact"
        assert np.array_equal(sel.cpu().numpy(), o_sel), "selection not bit-exact"
    else:
        fin = np.isfinite(o_bs)
        assert np.array_equal(np.isfinite(g_bs), fin)
        err = np.abs(g_bs[fin] - o_bs[fin]).max() if fin.any() else 0.0
        scale = np.abs(o_bs[fin]).max() if fin.any() else 1.0
        log(f"  block-score max abs err {err:.3e} (max |score| {scale:.3e})")
        assert err <= 1e-5 * scale
    assert np.array_equal(n_sel.cpu().numpy(), o_nsel)
    equal, n_diff = check_selection(sel.cpu().numpy(), o_sel, o_bs, gw.qs["pos"], n_sel.cpu().numpy())
    log(f"  selection: {equal.sum()} of {equal.size} (query, group) sets identical, {n_diff} near-tie swaps")
    # attention on the oracle's selection (all queries) and end to end
    o_out = oracle.sparse_attend(gw.host["k"], gw.host["v"], gw.qs["stream"], gw.qs["pos"], gw.qs["q"],
                                 o_sel, unit=128, scale=W.SCALE)
    out_o = _attend_gpu(gw, dims, dev(o_sel)).cpu().numpy()
    wa, wr = check_attention(out_o, o_out)
    log(f"  attention on the oracle selection: max-abs {wa:.3e}, rel-L2 {wr:.3e}")
    out_e2e = _attend_gpu(gw, dims, sel).cpu().numpy()
    check_attention(out_e2e, o_out, mask_qg=equal)
    # deterministic: a second run is bitwise identical
    out_again = _attend_gpu(gw, dims, sel).cpu().numpy()
    assert np.array_equal(out_e2e, out_again)
    sel2, _ = _select_gpu(gw, dims)
    assert torch.equal(sel, sel2)
    return gw


def test_decode_integer_1x4k_bitexact():
    gw = _decode_parity(W.CONFIGS["decode_1x4k_int"], exact=True)
    # and the stored fixture
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "decode_1x4k_int.txt")
    for line in open(path):
        if line.startswith("sel "):
            _, g, *ids = line.split()
            dims = M.msa_dims(16, W.SCALE)
            sel, _ = _select_gpu(gw, dims)
            assert sel[0, int(g)].tolist() == [int(x) for x in ids]


def test_decode_small_ragged_positions():
    # cap not a multiple of 128; positions at block edges, 0, partial local blocks
    pos = [0, 1, 127, 128, 129, 1000, 2047, 2048, 2049, 4095, 4999, 3333]
    wl = W.Workload("ragged", "msa_decode", 5, 5000, tuple(i % 5 for i in range(len(pos))), tuple(pos))
    _decode_parity(wl)


@pytest.mark.parametrize("top_k", [1, 5, 17, 64])
def test_decode_top_k_variants(top_k):
    pos = [0, 300, 2100, 8191, 6000]
    wl = W.Workload(f"topk{top_k}", "msa_decode", 2, 8192, (0, 1, 0, 1, 0), tuple(pos), top_k=top_k)
    _decode_parity(wl)


def test_decode_integer_ties_go_to_lower_block():
    # every index key equal: all visible blocks tie; local block + lowest ids
    wl = W.Workload("ties", "msa_decode", 1, 4096, (0, 0), (4095, 2500), idx_dist="int8")
    host = W.caches(wl)
    host["idx_k"][:] = 1.0
    gw = _decode_parity(wl, exact=True, host=host)
    dims = M.msa_dims(16, W.SCALE)
    sel, _ = _select_gpu(gw, dims)
    assert sel[0, 0].tolist() == list(range(15)) + [31]
    assert sel[1, 0].tolist() == list(range(15)) + [19]


def test_decode_full_32x32k():
    _decode_parity(W.CONFIGS["decode_32x32k"])


def test_decode_full_8x128k():
    _decode_parity(W.CONFIGS["decode_8x128k"])


def test_decode_max_context_4096_blocks():
    """The largest context the block top-k ranks: 4096 blocks (524288 keys)."""
    cap = 4096 * 128
    wl = W.Workload("max_ctx", "msa_decode", 1, cap, (0, 0, 0), (cap - 1, cap - 129, 300000))
    _decode_parity(wl)


def test_prefill_max_context_4096_blocks():
    """A prefill chunk ending at the last key of a 4096-block context."""
    cap = 4096 * 128
    _prefill_parity(W.prefill_workload("pf_max_ctx", cap, cap - 100, 100))


def test_empty_calls_launch_nothing():
    wl = W.decode_workload("e", 1, 256)
    gw = GpuWorkload(wl)
    dims = M.msa_dims()
    z = torch.empty(0, dtype=torch.int32, device=DEV)
    sel = torch.full((1, 4, 16), 7, dtype=torch.int32, device=DEV)
    n_sel = torch.full((1, 4), 7, dtype=torch.int32, device=DEV)
    M.msa_select(dims, gw.cache, dev(gw.qs["idx_q"]), z, z, 255, sel, n_sel, None)
    torch.cuda.synchronize()
    assert int(sel.sum()) == 7 * 64 and int(n_sel.sum()) == 28


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def _prefill_parity(wl: W.Workload, sample=None):
    log(f"[msa prefill] {wl.name}: cap={wl.cap} pos0={wl.pos[0]} n_q={wl.n_q}")
    dims = M.msa_dims(wl.top_k, W.SCALE)
    gw = GpuWorkload(wl)
    gw.append_own_rows()              # the whole chunk's keys, before its queries score
    n_q, pos0, s0 = wl.n_q, wl.pos[0], wl.stream[0]
    idx_q = dev(gw.qs["idx_q"])
    nblk = wl.max_pos // 128 + 1
    bs = torch.empty((n_q, 4, nblk), dtype=torch.float32, device=DEV)
    M.msa_block_scores_prefill(dims, gw.cache, idx_q, s0, pos0, bs, gw.ws(dims, M.MSA_OP_BLOCK_SCORES_PREFILL))
    sel = torch.empty((n_q, 4, wl.top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((n_q, 4), dtype=torch.int32, device=DEV)
    M.msa_select_prefill(dims, gw.cache, idx_q, s0, pos0, sel, n_sel,
                         gw.ws(dims, M.MSA_OP_SELECT_PREFILL))
    out = torch.empty((n_q, 64, 128), dtype=torch.float32, device=DEV)
    M.msa_attend_prefill(dims, gw.cache, gw.q, s0, pos0, sel, out, gw.ws(dims, M.MSA_OP_ATTEND_PREFILL))
    # the decode-form kernels on the same queries (unified selection semantics)
    sel_d, _ = _select_gpu(gw, dims)
    torch.cuda.synchronize()
    idx = np.arange(n_q) if sample is None else np.asarray(sample)
    o_bs, o_sel, o_nsel = oracle.msa_select(gw.host["idx_k"], gw.qs["stream"][idx], gw.qs["pos"][idx],
                                            gw.qs["idx_q"][idx], top_k=wl.top_k, nblk_out=nblk)
    g_bs = bs.cpu().numpy()[idx]
    fin = np.isfinite(o_bs)
    assert np.array_equal(np.isfinite(g_bs), fin)
    err = np.abs(g_bs[fin] - o_bs[fin]).max()
    log(f"  block-score max abs err {err:.3e} (max |score| {np.abs(o_bs[fin]).max():.3e})")
    assert err <= 1e-5 * np.abs(o_bs[fin]).max()
    g_sel = sel.cpu().numpy()[idx]
    assert np.array_equal(n_sel.cpu().numpy()[idx], o_nsel)
    equal, n_diff = check_selection(g_sel, o_sel, o_bs, gw.qs["pos"][idx])
    log(f"  selection: {equal.sum()} of {equal.size} identical, {n_diff} near-tie swaps")
    check_selection(sel_d.cpu().numpy()[idx], o_sel, o_bs, gw.qs["pos"][idx])
    o_out = oracle.sparse_attend(gw.host["k"], gw.host["v"], gw.qs["stream"][idx], gw.qs["pos"][idx],
                                 gw.qs["q"][idx], o_sel, unit=128, scale=W.SCALE)
    wa, wr = check_attention(out.cpu().numpy()[idx], o_out, mask_qg=equal)
    log(f"  attention end to end: max-abs {wa:.3e}, rel-L2 {wr:.3e}")
    # attention on the oracle selection, through the prefill entry point
    sel_o = sel.clone()
    sel_o[torch.from_numpy(idx).long().to(DEV)] = dev(o_sel)
    out2 = torch.empty_like(out)
    M.msa_attend_prefill(dims, gw.cache, gw.q, s0, pos0, sel_o, out2, gw.ws(dims, M.MSA_OP_ATTEND_PREFILL))
    check_attention(out2.cpu().numpy()[idx], o_out)


def test_prefill_small_ragged():
    # 300 queries: three 128-query tiles with a ragged tail; ragged cache
    _prefill_parity(W.prefill_workload("pf_small", 3000, 1900, 300))


def test_prefill_from_position_zero():
    _prefill_parity(W.prefill_workload("pf_zero", 700, 0, 700))


@pytest.mark.parametrize("top_k", [7, 64])
def test_prefill_second_stream_cache_edge(top_k):
    # stream 1 of 2; the last queries' local block runs past the cache end
    wl = W.Workload(f"pf_edge{top_k}", "msa_prefill", 2, 1000, tuple([1] * 100),
                    tuple(range(900, 1000)), idx_dist="normal_scaled", top_k=top_k)
    _prefill_parity(wl)


def test_prefill_attention_shared_selection():
    # every 16 consecutive queries share their 15 non-local blocks (the overlap
    # real text shows), so most staged blocks serve many queries at once
    wl = W.prefill_workload("pf_shared", 3000, 2500, 300)
    log(f"[msa prefill] {wl.name}: shared selections")
    dims = M.msa_dims(16, W.SCALE)
    gw = GpuWorkload(wl)
    gw.append_own_rows()
    n_q, pos0 = wl.n_q, wl.pos[0]
    rng = np.random.default_rng(7)
    loc = np.arange(pos0, pos0 + n_q) // 128
    sel = np.empty((n_q, 4, 16), np.int32)
    for t0 in range(0, n_q, 16):
        for g in range(4):
            others = rng.choice(pos0 // 128, 15, replace=False)
            for i in range(t0, min(t0 + 16, n_q)):
                sel[i, g] = np.sort(np.append(others, loc[i]))
    out = torch.empty((n_q, 64, 128), dtype=torch.float32, device=DEV)
    M.msa_attend_prefill(dims, gw.cache, gw.q, wl.stream[0], pos0, dev(sel), out, gw.ws(dims, M.MSA_OP_ATTEND_PREFILL))
    torch.cuda.synchronize()
    o_out = oracle.sparse_attend(gw.host["k"], gw.host["v"], gw.qs["stream"], gw.qs["pos"], gw.qs["q"], sel,
                                 unit=128, scale=W.SCALE)
    wa, wr = check_attention(out.cpu().numpy(), o_out)
    log(f"  attention: max-abs {wa:.3e}, rel-L2 {wr:.3e}")


@pytest.mark.parametrize("q_scale", [6.0, 40.0])
def test_prefill_attention_large_score_range(q_scale):
    # Queries scaled up so that block maxima run far above each query's first
    # reference: x6 moves the running reference, x40 also pushes scaled
    # probabilities past the overflow bound, so steps are recomputed.
    wl = W.prefill_workload(f"pf_big{int(q_scale)}", 3000, 2500, 200)
    log(f"[msa prefill] {wl.name}: queries scaled by {q_scale}")
    dims = M.msa_dims(16, W.SCALE)
    gw = GpuWorkload(wl)
    gw.append_own_rows()
    q32 = (gw.qs["q"].astype(np.uint32) << 16).view(np.float32) * np.float32(q_scale)
    qb = W.to_bf16_bits(q32)
    q_dev = dev_bits(qb, torch.bfloat16)
    n_q, pos0 = wl.n_q, wl.pos[0]
    rng = np.random.default_rng(11)
    sel = np.empty((n_q, 4, 16), np.int32)
    for i in range(n_q):
        loc = (pos0 + i) // 128
        for g in range(4):
            sel[i, g] = np.sort(np.append(rng.choice(loc, 15, replace=False), loc))
    out = torch.empty((n_q, 64, 128), dtype=torch.float32, device=DEV)
    M.msa_attend_prefill(dims, gw.cache, q_dev, wl.stream[0], pos0, dev(sel), out, gw.ws(dims, M.MSA_OP_ATTEND_PREFILL))
    torch.cuda.synchronize()
    o_out = oracle.sparse_attend(gw.host["k"], gw.host["v"], gw.qs["stream"], gw.qs["pos"], qb, sel,
                                 unit=128, scale=W.SCALE)
    wa, wr = check_attention(out.cpu().numpy(), o_out)
    log(f"  attention: max-abs {wa:.3e}, rel-L2 {wr:.3e}")


def test_prefill_full_4096_at_32k():
    """The whole 4096-query chunk at 32K, every query: block scores, the
    selection under the near-tie rule (prefill and decode kernels), attention
    end to end and on the oracle's own selection."""
    _prefill_parity(W.CONFIGS["prefill_4096_at_32k"])


def test_decode_step_graph_replay_matches_eager():
    """A captured decode step (append, select, attend) replayed several times,
    with eager work and synchronisations in between, reproduces the eager
    result bit for bit every time (no memset nodes are recorded)."""
    wl = W.decode_workload("graph", 4, 3000)
    dims = M.msa_dims(16, W.SCALE)
    gw = GpuWorkload(wl)
    h, qs = gw.host, gw.qs
    s_np, p_np = qs["stream"], qs["pos"]
    new_idx = dev(h["idx_k"][s_np, p_np])
    from _gpu_common import dev_bits
    new_k = dev_bits(h["k"][s_np, p_np], torch.bfloat16)
    new_v = dev_bits(h["v"][s_np, p_np], torch.bfloat16)
    idx_q = dev(qs["idx_q"])
    sel = torch.empty((4, 4, 16), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((4, 4), dtype=torch.int32, device=DEV)
    out = torch.empty((4, 64, 128), dtype=torch.float32, device=DEV)
    ws_s = gw.ws(dims, M.MSA_OP_SELECT)
    ws_a = gw.ws(dims, M.MSA_OP_ATTEND_DECODE)

    def step():
        M.msa_index_append(dims, gw.cache, gw.stream, gw.pos, wl.max_pos, new_idx, new_k, new_v)
        M.msa_select(dims, gw.cache, idx_q, gw.stream, gw.pos, wl.max_pos, sel, n_sel, ws_s)
        M.msa_attend_decode(dims, gw.cache, gw.q, gw.stream, gw.pos, wl.max_pos, sel, out, ws_a)

    step()
    torch.cuda.synchronize()
    ref_out, ref_sel = out.clone(), sel.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(6):
        out.zero_()
        sel.fill_(-7)
        # the attention workspace is cleared before some replays only: the
        # split counter must also start over from what the last replay (same
        # launch tag) or an eager call (another tag) left in it
        if r == 0:
            ws_a.zero_()
        elif r == 3:
            step()
            out.zero_()
            sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel), f"replay {r}: selection differs"
        assert torch.equal(out, ref_out), f"replay {r}: output differs"
        _ = (out * 2).sum().item()      # eager work between replays
