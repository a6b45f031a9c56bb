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

    wa, wr = check_attention(attend(dev(o_sel)), o_out)
    log(f"  attention on the oracle selection: max-abs {wa:.3e}, rel-L2 {wr:.3e}")
    check_attention(attend(sel), o_out, mask_qg=np.repeat(equal[:, None], 4, 1))


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
