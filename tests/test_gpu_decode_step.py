"""GPU tests of msa_decode_step (append, selection and attention of one
decode step in one call), through the C ABI.

Its outputs -- the appended cache rows, the selection, its sizes and the
attention output -- must equal those of msa_index_append + msa_select +
msa_attend_decode bit for bit: on the three-kernel form (few queries over
at most 64 blocks, f32 index cache, bf16 K/V: the scan appends the rows and
scores the new keys from the inputs, the attention ranks the blocks itself,
then the split combine, or, after the fine scan, the last split of each
(query, group) merging the partials itself) and on the separate-kernel form
the other shapes take.  The integer workload
is also held to the oracle (selection bit-exact, attention to the attention
tolerances), and queries of one stream at neighbouring positions score each
other's new keys.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W
from _gpu_common import DEV, check_attention, dev, dev_bits, log

pytestmark = pytest.mark.gpu


def _both_forms(wl: W.Workload, paged: bool = False):
    """Runs the step both ways on identical caches (the step's own rows
    zeroed first, so both must write them); returns the step's outputs."""
    host, qs = W.caches(wl), W.queries(wl)
    dims = M.msa_dims(wl.top_k, W.SCALE)
    st, ps = qs["stream"].astype(np.int64), qs["pos"].astype(np.int64)
    assert len(set(zip(st.tolist(), ps.tolist()))) == wl.n_q, "the step's (stream, pos) pairs must be distinct"
    new_idx = dev(host["idx_k"][st, ps])
    new_k = dev_bits(host["k"][st, ps], torch.bfloat16)
    new_v = dev_bits(host["v"][st, ps], torch.bfloat16)
    q, idx_q = dev_bits(qs["q"], torch.bfloat16), dev(qs["idx_q"])
    stream, pos = dev(qs["stream"]), dev(qs["pos"])
    S, cap = wl.n_stream, wl.cap
    nb = (cap + 127) // 128
    table = np.random.default_rng(11).permutation(S * nb + 3)[: S * nb].astype(np.int32).reshape(S, nb)
    results = []
    for fused in (False, True):
        idx_k = dev(host["idx_k"])
        k = dev_bits(host["k"], torch.bfloat16)
        v = dev_bits(host["v"], torch.bfloat16)
        ti, tp = torch.from_numpy(st), torch.from_numpy(ps)
        idx_k[ti, tp] = 0
        k[ti, tp] = 0
        v[ti, tp] = 0
        if paged:
            # the same rows placed in pages by a seeded table
            n_pages = S * nb + 3
            pk = torch.zeros((n_pages * 128, 4, 128), dtype=torch.bfloat16, device=DEV)
            pv, pi = torch.zeros_like(pk), torch.zeros((n_pages * 128, 4, 128), dtype=torch.float32, device=DEV)
            for s in range(S):
                for b in range(nb):
                    r0, r1 = b * 128, min(cap, b * 128 + 128)
                    d0 = int(table[s, b]) * 128
                    pk[d0:d0 + r1 - r0] = k[s, r0:r1]
                    pv[d0:d0 + r1 - r0] = v[s, r0:r1]
                    pi[d0:d0 + r1 - r0] = idx_k[s, r0:r1]
            k, v, idx_k = pk, pv, pi
            cache = M.make_cache(k=k, v=v, idx_k=idx_k, block_table=dev(table), cap=cap)
        else:
            cache = M.make_cache(k=k, v=v, idx_k=idx_k)
        sel = torch.full((wl.n_q, 4, wl.top_k), -7, dtype=torch.int32, device=DEV)
        n_sel = torch.full((wl.n_q, 4), -7, dtype=torch.int32, device=DEV)
        out = torch.zeros((wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
        if fused:
            ws = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_DECODE_STEP, wl.n_q, wl.max_pos), 256),
                             dtype=torch.uint8, device=DEV)
            M.msa_decode_step(dims, cache, stream, pos, wl.max_pos, new_idx, new_k, new_v, idx_q, q, sel, n_sel,
                              out, ws)
        else:
            M.msa_index_append(dims, cache, stream, pos, wl.max_pos, idx_k_new=new_idx, k_new=new_k, v_new=new_v)
            ws_s = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_SELECT, wl.n_q, wl.max_pos), 256),
                               dtype=torch.uint8, device=DEV)
            M.msa_select(dims, cache, idx_q, stream, pos, wl.max_pos, sel, n_sel, ws_s)
            ws_a = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_ATTEND_DECODE, wl.n_q, wl.max_pos), 256),
                               dtype=torch.uint8, device=DEV)
            M.msa_attend_decode(dims, cache, q, stream, pos, wl.max_pos, sel, out, ws_a)
        torch.cuda.synchronize()
        results.append({"idx_k": idx_k.cpu(), "k": k.view(torch.int16).cpu(), "v": v.view(torch.int16).cpu(),
                        "sel": sel.cpu(), "n_sel": n_sel.cpu(), "out": out.cpu()})
    for name in results[0]:
        assert torch.equal(results[0][name], results[1][name]), f"{name}: the step differs from the separate calls"
    assert torch.isfinite(results[1]["out"]).all()
    return results[1], host, qs


# Shapes: the three-kernel form takes an f32 index cache, bf16 K/V and at
# most 1024 blocks; its scan is the fine one (partial maxima) when
# n_q * ceil(nblk / 2) < 256, and the attention ranks up to 64 blocks
# directly, more by register rounds (4, 8 or 16 keys per lane).
CASES = [
    # (name, n_stream, cap, streams, positions, top_k)
    ("one_query_4k", 1, 4096, (0,), (4095,), 16),
    ("ragged_5", 5, 3000, (0, 1, 2, 3, 4), (2999, 0, 127, 128, 1500), 16),
    ("one_stream_neighbours", 2, 3000, (0, 0, 0, 1, 0), (1000, 1001, 1130, 500, 1127), 16),
    ("short_top64", 3, 8192, (0, 1, 2), (200, 8191, 4000), 64),
    ("top1", 2, 2048, (0, 1), (2047, 300), 1),
    ("coarse_scan_20x8k", 20, 8192, tuple(range(20)), tuple(8191 - 37 * j for j in range(20)), 16),
    ("fine_scan_register_rank", 2, 20000, (0, 1), (19999, 9000), 16),
    ("coarse_scan_one_stream_neighbours", 3, 40000, (0, 0, 1, 0, 2), (39999, 39998, 20000, 30000, 128), 16),
    ("coarse_scan_1024_blocks", 1, 131072, (0,), (131071,), 16),
    ("separate_kernels_over_1024_blocks", 1, 140000, (0,), (139999,), 16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_step_equals_separate_calls(case):
    name, S, cap, streams, positions, top_k = case
    wl = W.Workload(f"step_{name}", "msa_decode", S, cap, streams, positions, top_k=top_k)
    log(f"[decode step] {name}: n_q={wl.n_q} max_pos={wl.max_pos} top_k={top_k}")
    _both_forms(wl)


def test_decode_step_paged():
    wl = W.Workload("step_paged", "msa_decode", 3, 3000, (0, 1, 2, 1), (2999, 1500, 130, 1501), top_k=16)
    log("[decode step] paged cache")
    _both_forms(wl, paged=True)


def test_decode_step_integer_workload_against_oracle():
    """The 1 x 4K integer-indexer decode: the step's selection equals the
    oracle's bit for bit, its attention is within the attention tolerances."""
    wl = W.CONFIGS["decode_1x4k_int"]
    log(f"[decode step] {wl.name} against the oracle")
    res, host, qs = _both_forms(wl)
    _, o_sel, o_nsel = oracle.msa_select(host["idx_k"], qs["stream"], qs["pos"], qs["idx_q"], top_k=wl.top_k)
    assert np.array_equal(res["sel"].numpy(), o_sel)
    assert np.array_equal(res["n_sel"].numpy(), o_nsel)
    o_out = oracle.sparse_attend(host["k"], host["v"], qs["stream"], qs["pos"], qs["q"], o_sel, unit=128,
                                 scale=W.SCALE)
    wa, wr = check_attention(res["out"].numpy(), o_out)
    log(f"  attention max-abs {wa:.3e}, rel-L2 {wr:.3e}")


@pytest.mark.parametrize("ctx,n_stream", [(4096, 1), (16384, 24)])
def test_decode_step_graph_replay_matches_eager(ctx, n_stream):
    """msa_decode_step captured into a HIP graph and replayed six times, with
    eager work and synchronisations in between (outputs cleared, the
    workspace cleared before one replay, an eager call before another),
    reproduces the eager step bit for bit every time: the fine-scan form
    (one query over 4096 slots) and the regular-scan form (24 queries over
    16384)."""
    wl = W.decode_workload(f"step_graph_{ctx}", n_stream, ctx)
    host, qs = W.caches(wl), W.queries(wl)
    dims = M.msa_dims(16, W.SCALE)
    st, ps = qs["stream"].astype(np.int64), qs["pos"].astype(np.int64)
    cache = M.make_cache(k=dev_bits(host["k"], torch.bfloat16), v=dev_bits(host["v"], torch.bfloat16),
                         idx_k=dev(host["idx_k"]))
    stream, pos = dev(qs["stream"]), dev(qs["pos"])
    new_idx = dev(host["idx_k"][st, ps])
    new_k = dev_bits(host["k"][st, ps], torch.bfloat16)
    new_v = dev_bits(host["v"][st, ps], torch.bfloat16)
    idx_q, q = dev(qs["idx_q"]), dev_bits(qs["q"], torch.bfloat16)
    sel = torch.empty((wl.n_q, 4, 16), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((wl.n_q, 4), dtype=torch.int32, device=DEV)
    out = torch.empty((wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(M.workspace_bytes(dims, M.MSA_OP_DECODE_STEP, wl.n_q, wl.max_pos), dtype=torch.uint8,
                     device=DEV)
    log(f"[decode step] graph replay: {wl.n_q} queries over {ctx} slots")

    def step():
        M.msa_decode_step(dims, cache, stream, pos, wl.max_pos, new_idx, new_k, new_v, idx_q, q, sel, n_sel, out, ws)

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
            ws.zero_()
        elif r == 3:
            step()
            out.zero_()
            sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: output differs"
        assert torch.equal(sel, ref_sel) and torch.equal(n_sel, ref_n), f"replay {r}: selection differs"


@pytest.mark.parametrize("fmt", ["f16_index", "int8_kv", "q4_kv"])
def test_decode_step_other_cache_formats(fmt):
    """msa_decode_step on an fp16 index cache, and on int8 and 4-bit K/V
    caches (the separate calls' kernels inside one call), equals
    msa_index_append + msa_select + msa_attend_decode bit for bit: the rows
    it appends (codes and scales included), the selection and the output.
    Every cache row is first written through the append entry point; the
    step's own rows are then zeroed, so both forms must write them."""
    wl = W.Workload(f"step_{fmt}", "msa_decode", 3, 3000, (0, 1, 2, 1), (2999, 1500, 130, 700))
    log(f"[decode step] {fmt}: n_q={wl.n_q} max_pos={wl.max_pos}")
    host, qs = W.caches(wl), W.queries(wl)
    dims = M.msa_dims(wl.top_k, W.SCALE)
    S, cap = wl.n_stream, wl.cap
    st, ps = qs["stream"].astype(np.int64), qs["pos"].astype(np.int64)
    ti, tp = torch.from_numpy(st), torch.from_numpy(ps)
    kv_format = {"f16_index": M.KV_BF16, "int8_kv": M.KV_INT8, "q4_kv": M.KV_Q4}[fmt]
    new_idx = dev(host["idx_k"][st, ps])
    new_k = dev_bits(host["k"][st, ps], torch.bfloat16)
    new_v = dev_bits(host["v"][st, ps], torch.bfloat16)
    q, idx_q = dev_bits(qs["q"], torch.bfloat16), dev(qs["idx_q"])
    stream, pos = dev(qs["stream"]), dev(qs["pos"])
    all_st = torch.arange(S, dtype=torch.int32, device=DEV).repeat_interleave(cap)
    all_ps = torch.arange(cap, dtype=torch.int32, device=DEV).repeat(S)
    results = []
    for fused in (False, True):
        t = {}
        if fmt == "f16_index":
            t["idx_k_f16"] = torch.zeros((S, cap, 4, 128), dtype=torch.float16, device=DEV)
        else:
            t["idx_k"] = torch.zeros((S, cap, 4, 128), dtype=torch.float32, device=DEV)
        if kv_format == M.KV_BF16:
            t["k"] = torch.zeros((S, cap, 4, 128), dtype=torch.bfloat16, device=DEV)
        else:
            t["k"] = torch.zeros((S, cap, 4, 128 if kv_format == M.KV_INT8 else 64), dtype=torch.uint8, device=DEV)
            t["k_scale"] = torch.zeros((S, cap, 4, 4), dtype=torch.float32, device=DEV)
            t["v_scale"] = torch.zeros_like(t["k_scale"])
        t["v"] = torch.zeros_like(t["k"])
        cache = M.make_cache(kv_format=kv_format, **t)
        M.msa_index_append(dims, cache, all_st, all_ps, cap - 1, idx_k_new=dev(host["idx_k"].reshape(S * cap, 4, 128)),
                           k_new=dev_bits(host["k"].reshape(S * cap, 4, 128), torch.bfloat16),
                           v_new=dev_bits(host["v"].reshape(S * cap, 4, 128), torch.bfloat16))
        for name in t:
            t[name][ti, tp] = 0
        sel = torch.full((wl.n_q, 4, wl.top_k), -7, dtype=torch.int32, device=DEV)
        n_sel = torch.full((wl.n_q, 4), -7, dtype=torch.int32, device=DEV)
        out = torch.zeros((wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
        if fused:
            ws = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_DECODE_STEP, wl.n_q, wl.max_pos), 256),
                             dtype=torch.uint8, device=DEV)
            M.msa_decode_step(dims, cache, stream, pos, wl.max_pos, new_idx, new_k, new_v, idx_q, q, sel, n_sel,
                              out, ws)
        else:
            M.msa_index_append(dims, cache, stream, pos, wl.max_pos, idx_k_new=new_idx, k_new=new_k, v_new=new_v)
            ws_s = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_SELECT, wl.n_q, wl.max_pos), 256),
                               dtype=torch.uint8, device=DEV)
            M.msa_select(dims, cache, idx_q, stream, pos, wl.max_pos, sel, n_sel, ws_s)
            ws_a = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_ATTEND_DECODE, wl.n_q, wl.max_pos), 256),
                               dtype=torch.uint8, device=DEV)
            M.msa_attend_decode(dims, cache, q, stream, pos, wl.max_pos, sel, out, ws_a)
        torch.cuda.synchronize()
        r = {name: (x.view(torch.int16) if x.dtype in (torch.bfloat16, torch.float16) else x).cpu()
             for name, x in t.items()}
        r.update(sel=sel.cpu(), n_sel=n_sel.cpu(), out=out.cpu())
        results.append(r)
    for name in results[0]:
        assert torch.equal(results[0][name], results[1][name]), f"{name}: the step differs from the separate calls"
    assert torch.isfinite(results[1]["out"]).all()
    assert (results[1]["n_sel"] > 0).all()
