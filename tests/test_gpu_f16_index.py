"""GPU parity of the fp16 index-key cache (msa_cache.idx_k_f16) against the
fp64 oracle, through the C ABI.

The append rounds the f32 keys it receives to fp16 (nearest, ties to even),
which must equal numpy's float32 -> float16 conversion bit for bit.  The block
scores and the top-16 selection must then match the oracle evaluated on the
fp16-rounded keys (widened exactly to f32), under the same rules as the f32
cache: bit-exact on integer-valued keys (exact in fp16), the near-tie rule on
Gaussian ones.  Attention reads only K/V and is unaffected by the index
cache type.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W
from _gpu_common import DEV, check_selection, dev, dev_bits, host_bits, log

pytestmark = pytest.mark.gpu


def _f16_case(wl: W.Workload, exact: bool = False):
    log(f"[f16 index] {wl.name}: kind={wl.kind} streams={wl.n_stream} cap={wl.cap} n_q={wl.n_q}")
    host = W.caches(wl)
    qs = W.queries(wl)
    k16_host = host["idx_k"].astype(np.float16)            # round to nearest even
    keys = k16_host.astype(np.float32)                     # exact: what the index cache holds
    dims = M.msa_dims(wl.top_k, W.SCALE)
    idx16 = torch.from_numpy(k16_host).to(DEV)
    k = dev_bits(host["k"], torch.bfloat16)
    v = dev_bits(host["v"], torch.bfloat16)
    cache = M.make_cache(k=k, v=v, idx_k_f16=idx16)

    # append: the queries' own rows are cleared and written from the f32 keys
    pairs = sorted(set(zip(wl.stream, wl.pos)))
    s_arr = np.array([a for a, _ in pairs], np.int32)
    p_arr = np.array([b for _, b in pairs], np.int32)
    si, pi = torch.from_numpy(s_arr).long(), torch.from_numpy(p_arr).long()
    idx16[si, pi] = 0
    M.msa_index_append(dims, cache, dev(s_arr), dev(p_arr), int(p_arr.max()),
                       idx_k_new=dev(host["idx_k"][s_arr, p_arr]))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(idx16[si, pi]), k16_host[s_arr, p_arr].view(np.uint16)), \
        "fp16 append differs from round-to-nearest-even"

    n_q = wl.n_q
    nblk = wl.max_pos // 128 + 1
    idx_q = dev(qs["idx_q"])
    stream, pos = dev(qs["stream"]), dev(qs["pos"])
    sel = torch.empty((n_q, 4, wl.top_k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((n_q, 4), dtype=torch.int32, device=DEV)
    bs = torch.empty((n_q, 4, nblk), dtype=torch.float32, device=DEV)
    ws = lambda op, mp=wl.max_pos: torch.empty(max(M.workspace_bytes(dims, op, n_q, mp), 256),
                                               dtype=torch.uint8, device=DEV)
    if wl.kind == "msa_prefill":
        s0, pos0 = wl.stream[0], wl.pos[0]
        M.msa_block_scores_prefill(dims, cache, idx_q, s0, pos0, bs, ws(M.MSA_OP_BLOCK_SCORES_PREFILL))
        M.msa_select_prefill(dims, cache, idx_q, s0, pos0, sel, n_sel, ws(M.MSA_OP_SELECT_PREFILL))
    else:
        M.msa_block_scores(dims, cache, idx_q, stream, pos, wl.max_pos, bs)
        M.msa_select(dims, cache, idx_q, stream, pos, wl.max_pos, sel, n_sel, ws(M.MSA_OP_SELECT))
    torch.cuda.synchronize()
    o_bs, o_sel, o_nsel = oracle.msa_select(keys, qs["stream"], qs["pos"], qs["idx_q"], top_k=wl.top_k,
                                            nblk_out=nblk)
    g_bs = bs.cpu().numpy()
    if exact:
        assert np.array_equal(g_bs.astype(np.float64), o_bs), "block scores not bit-exact"
        assert np.array_equal(sel.cpu().numpy(), o_sel), "selection not bit-exact"
    else:
        fin = np.isfinite(o_bs)
        assert np.array_equal(np.isfinite(g_bs), fin)
        err = np.abs(g_bs[fin] - o_bs[fin]).max()
        scale = np.abs(o_bs[fin]).max()
        log(f"  block-score max abs err {err:.3e} (max |score| {scale:.3e})")
        assert err <= 1e-5 * scale
    assert np.array_equal(n_sel.cpu().numpy(), o_nsel)
    equal, n_diff = check_selection(sel.cpu().numpy(), o_sel, o_bs, qs["pos"], n_sel.cpu().numpy())
    log(f"  selection: {equal.sum()} of {equal.size} (query, group) sets identical, {n_diff} near-tie swaps")


def test_f16_index_decode_integer_1x4k_bitexact():
    _f16_case(W.CONFIGS["decode_1x4k_int"], exact=True)


def test_f16_index_decode_small_ragged_positions():
    pos = [0, 1, 127, 128, 129, 1000, 2047, 2048, 2049, 4095, 4999, 3333]
    _f16_case(W.Workload("ragged16", "msa_decode", 5, 5000, tuple(i % 5 for i in range(len(pos))), tuple(pos)))


def test_f16_index_decode_full_32x32k():
    _f16_case(W.CONFIGS["decode_32x32k"])


def test_f16_index_prefill_small_ragged():
    _f16_case(W.prefill_workload("pf16_small", 3000, 1900, 300))


def test_f16_index_prefill_from_position_zero():
    _f16_case(W.prefill_workload("pf16_zero", 700, 0, 700))
