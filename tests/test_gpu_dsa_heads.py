"""GPU parity of the multi-head DSA indexer (dsa_select_heads) against the fp64
oracle, through the C ABI.

score(i, j) = sum_h w[i][h] * max(0, q[i][h] . k[j]) over the rotated fp16 key
cache (fp16 products exact, f32 sums on the matrix cores), then the top-k of
dsa_select.  The scores, which the call leaves in its workspace, are compared
with the oracle's to 2e-6 of the largest |score| (f32 sums of 128 exact
products per head and 16-64 heads); the selection under the near-tie rule
(sets equal, or differing only in keys within 1e-5 * max|score| of the
oracle's boundary score); attention over the selection to the attention
tolerances.  IndexShare: a second layer attends with the first layer's
selection.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W
from _gpu_common import DEV, GpuWorkload, check_attention, check_token_selection, dev, dev_bits, host_bits, log

pytestmark = pytest.mark.gpu

SCORE_REL = 2e-6


def _score_stride(max_pos):
    return ((max_pos + 1 + 63) // 64) * 64


def _heads_case(wl: W.Workload, n_head: int, check_attend: bool = True):
    log(f"[dsa heads] {wl.name}: streams={wl.n_stream} cap={wl.cap} n_q={wl.n_q} heads={n_head} "
        f"top_k={wl.top_k}")
    dims = M.dsa_dims(wl.top_k, W.SCALE)
    gw = GpuWorkload(wl)
    gw.append_own_rows()
    torch.cuda.synchronize()
    o_rot = oracle.dsa_rotate(gw.host["dsa_k"])
    assert np.array_equal(host_bits(gw.dsa_k), o_rot), "rotated key cache differs from the oracle's"
    qh = W.queries_dsa_heads(wl, n_head)
    sel = torch.empty((wl.n_q, wl.top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty(wl.n_q, dtype=torch.int32, device=DEV)
    ws = gw.ws(dims, M.DSA_OP_SELECT)
    M.dsa_select_heads(dims, gw.cache, dev_bits(qh["q_idx_h"], torch.float16), dev(qh["head_w"]), gw.stream,
                       gw.pos, wl.max_pos, sel, n_sel, ws)
    torch.cuda.synchronize()
    o_sel, o_nsel, scores = oracle.dsa_select_heads(o_rot, gw.qs["stream"], gw.qs["pos"], qh["q_idx_h"],
                                                    qh["head_w"], top_k=wl.top_k, want_scores=True)
    # scores: the workspace holds [n_q][stride] f32
    stride = _score_stride(wl.max_pos)
    g_sc = ws[: wl.n_q * stride * 4].view(torch.float32).view(wl.n_q, stride).cpu().numpy()
    worst = 0.0
    for i, p in enumerate(gw.qs["pos"]):
        ref = scores[i, :p + 1]
        err = np.abs(g_sc[i, :p + 1] - ref).max() / max(np.abs(ref).max(), 1e-30)
        worst = max(worst, err)
        assert err <= SCORE_REL, f"query {i}: score error {err:.3e} of max |score|"
    equal = check_token_selection(sel.cpu().numpy(), n_sel.cpu().numpy(), o_sel, o_nsel, scores,
                                   gw.qs["pos"], wl.top_k)
    log(f"  scores: worst error {worst:.2e} of max |score|; selection: {equal.sum()} of {len(equal)} identical")
    if check_attend:
        o_out = oracle.sparse_attend(gw.host["k"], gw.host["v"], gw.qs["stream"], gw.qs["pos"], gw.qs["q"],
                                     o_sel, unit=1, scale=W.SCALE, shared_across_groups=True)
        out = torch.empty((wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
        M.dsa_attend_decode(dims, gw.cache, gw.q, gw.stream, gw.pos, wl.max_pos, sel, out,
                            gw.ws(dims, M.DSA_OP_ATTEND_DECODE))
        torch.cuda.synchronize()
        wa, wr = check_attention(out.cpu().numpy(), o_out, mask_qg=np.repeat(equal[:, None], 4, 1))
        log(f"  attention: max-abs {wa:.3e}, rel-L2 {wr:.3e}")
    return gw, sel, o_sel


_RAGGED = (4999, 3000, 127, 0, 2100, 64, 65, 1023, 1024, 4095)


@pytest.mark.parametrize("n_head", [16, 32, 48, 64])
def test_dsa_heads_ragged_positions(n_head):
    wl = W.Workload(f"dsa_heads_{n_head}", "dsa_decode", 3, 5000, tuple(i % 3 for i in range(len(_RAGGED))),
                    _RAGGED, top_k=64)
    _heads_case(wl, n_head)


def test_dsa_heads_short_context_keeps_everything():
    wl = W.Workload("dsa_heads_short", "dsa_decode", 2, 3000, (0, 1, 0), (2999, 1500, 2047), top_k=2048)
    _heads_case(wl, 32)


def test_dsa_heads_full_16x64k():
    _heads_case(W.CONFIGS["dsa_16x64k"], W.DSA_N_IHEAD, check_attend=False)


def test_dsa_heads_index_share():
    """IndexShare: a shared layer reuses the previous full layer's top-k; its
    attention runs on its own K/V with that selection."""
    wl = W.Workload("dsa_share", "dsa_decode", 2, 4000, (0, 1, 1), (3999, 2500, 999), top_k=256)
    _, sel, o_sel = _heads_case(wl, 32, check_attend=False)
    wl2 = W.Workload("dsa_share", "dsa_decode", 2, 4000, (0, 1, 1), (3999, 2500, 999), top_k=256, seed=1)
    gw2 = GpuWorkload(wl2)               # the shared layer: other K/V, no index keys needed
    dims = M.dsa_dims(wl.top_k, W.SCALE)
    out = torch.empty((wl.n_q, 64, 128), dtype=torch.float32, device=DEV)
    M.dsa_attend_decode(dims, gw2.cache, gw2.q, gw2.stream, gw2.pos, wl.max_pos, dev(o_sel), out,
                        gw2.ws(dims, M.DSA_OP_ATTEND_DECODE))
    torch.cuda.synchronize()
    o_out = oracle.sparse_attend(gw2.host["k"], gw2.host["v"], gw2.qs["stream"], gw2.qs["pos"], gw2.qs["q"],
                                 o_sel, unit=1, scale=W.SCALE, shared_across_groups=True)
    wa, wr = check_attention(out.cpu().numpy(), o_out)
    log(f"  shared layer on the full layer's selection: max-abs {wa:.3e}, rel-L2 {wr:.3e}")
