"""Shared set-up for the GPU parity tests: upload seeded workloads, run the
HIP path through the Python binding of the C ABI, and compare with the oracle
under the tolerances the method fixes.

Tolerances:
  * integer, byte and index results: bit-exact;
  * block selection on Gaussian inputs: identical sets, except blocks whose
    oracle score lies within 1e-5 * max|score| of the oracle's boundary score
    (the k-th ranked block), i.e. the 16th/17th near-tie rule;
  * attention outputs: max-abs <= 1e-2 and relative L2 <= 5e-3 against the
    fp64 oracle, per query.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W

DEV = torch.device("cuda", 0)
ATOL_MAX = 1e-2
RTOL_L2 = 5e-3
GAP_REL = 1e-5


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bits(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """uint16 bit patterns -> device tensor of dtype (bf16 / f16)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dtype).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


class GpuWorkload:
    """Device caches of a workload.  The rows at the queries' own positions
    are first overwritten with zeros and then written by the append entry
    point, so the append is exercised on every run."""

    def __init__(self, wl: W.Workload, host=None):
        self.wl = wl
        self.host = W.caches(wl) if host is None else host
        self.qs = W.queries(wl)
        h = self.host
        self.k = dev_bits(h["k"], torch.bfloat16)
        self.v = dev_bits(h["v"], torch.bfloat16)
        self.dsa = wl.kind == "dsa_decode"
        if self.dsa:
            self.dsa_k = torch.zeros(h["dsa_k"].shape, dtype=torch.float16, device=DEV)
            self.idx_k = None
        else:
            self.idx_k = dev(h["idx_k"])
            self.dsa_k = None
        self.cache = M.make_cache(k=self.k, v=self.v, idx_k=self.idx_k, dsa_k=self.dsa_k)
        self.stream = dev(self.qs["stream"])
        self.pos = dev(self.qs["pos"])
        self.q = dev_bits(self.qs["q"], torch.bfloat16)
        self.max_pos = wl.max_pos

    def append_own_rows(self):
        """Write each query's own slot through the append entry point (DSA:
        every slot, since the rotated cache only exists on the device)."""
        wl, h = self.wl, self.host
        if self.dsa:
            S, cap = h["dsa_k"].shape[:2]
            st = torch.arange(S, dtype=torch.int32, device=DEV).repeat_interleave(cap)
            ps = torch.arange(cap, dtype=torch.int32, device=DEV).repeat(S)
            keys = dev_bits(h["dsa_k"].reshape(S * cap, -1), torch.float16)
            M.dsa_index_append(M.dsa_dims(wl.top_k), self.cache, st, ps, cap - 1, keys)
            return
        st, ps = self.qs["stream"], self.qs["pos"]
        # distinct (stream, pos) rows
        pairs = sorted(set(zip(st.tolist(), ps.tolist())))
        s_arr = np.array([a for a, _ in pairs], np.int32)
        p_arr = np.array([b for _, b in pairs], np.int32)
        si, pi = torch.from_numpy(s_arr).long(), torch.from_numpy(p_arr).long()
        self.idx_k[si, pi] = 0
        self.k[si, pi] = 0
        self.v[si, pi] = 0
        M.msa_index_append(M.msa_dims(wl.top_k), self.cache, dev(s_arr), dev(p_arr), int(p_arr.max()),
                           idx_k_new=dev(h["idx_k"][s_arr, p_arr]),
                           k_new=dev_bits(h["k"][s_arr, p_arr], torch.bfloat16),
                           v_new=dev_bits(h["v"][s_arr, p_arr], torch.bfloat16))

    def ws(self, dims, op, n_q=None, max_pos=None):
        n = M.workspace_bytes(dims, op, self.wl.n_q if n_q is None else n_q,
                              self.max_pos if max_pos is None else max_pos)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)


def check_selection(gpu_sel, orc_sel, orc_bs, pos, n_sel_gpu=None, n_sel_orc=None, block=128):
    """MSA: per (query, group) set equality up to near-ties at the boundary.
    Returns the boolean mask [n_q][G] of (query, group) whose sets are equal."""
    n_q, G, K = orc_sel.shape
    equal = np.zeros((n_q, G), bool)
    n_diff = 0
    for i in range(n_q):
        loc = pos[i] // block
        for g in range(G):
            a = set(int(x) for x in gpu_sel[i, g] if x >= 0)
            b = set(int(x) for x in orc_sel[i, g] if x >= 0)
            assert len(a) == len(b) == min(K, loc + 1), (i, g, len(a), len(b))
            assert loc in a, (i, g)
            ids = [x for x in gpu_sel[i, g] if x >= 0]
            assert ids == sorted(ids) and np.all(gpu_sel[i, g, len(ids):] == -1), (i, g)
            if n_sel_gpu is not None:
                assert n_sel_gpu[i, g] == len(a)
            if a == b:
                equal[i, g] = True
                continue
            n_diff += 1
            bs = orc_bs[i, g, :loc + 1]
            thr = GAP_REL * np.max(np.abs(bs[np.isfinite(bs)]))
            nonlocal_sel = [x for x in b if x != loc]
            boundary = min(bs[x] for x in nonlocal_sel)
            for x in a ^ b:
                assert abs(bs[x] - boundary) < thr, (
                    f"query {i} group {g}: block {x} (score {bs[x]}) differs beyond the near-tie "
                    f"band around {boundary} (thr {thr})")
    return equal, n_diff


def check_attention(got: np.ndarray, ref: np.ndarray, mask_qg=None, heads_per_group=16):
    """got, ref: [n_q][H][D]; mask_qg: [n_q][G] which (query, group) to compare."""
    got = got.astype(np.float64)
    n_q = got.shape[0]
    worst_abs, worst_rel = 0.0, 0.0
    for i in range(n_q):
        if mask_qg is None:
            hm = np.ones(got.shape[1], bool)
        else:
            hm = np.repeat(mask_qg[i], heads_per_group)
        if not hm.any():
            continue
        d = got[i, hm] - ref[i, hm]
        assert np.all(np.isfinite(got[i, hm])), f"query {i}: non-finite output"
        ma = np.abs(d).max()
        rel = np.linalg.norm(d) / max(np.linalg.norm(ref[i, hm]), 1e-30)
        worst_abs, worst_rel = max(worst_abs, ma), max(worst_rel, rel)
        assert ma <= ATOL_MAX, f"query {i}: max-abs {ma}"
        assert rel <= RTOL_L2, f"query {i}: rel-L2 {rel}"
    return worst_abs, worst_rel


def check_token_selection(g_sel, g_nsel, o_sel, o_nsel, scores, pos, top_k):
    equal = np.zeros(len(pos), bool)
    for i in range(len(pos)):
        k = min(top_k, pos[i] + 1)
        assert g_nsel[i] == o_nsel[i] == k
        ids = g_sel[i, :k]
        assert np.all(np.diff(ids) > 0) and ids.min() >= 0 and ids.max() <= pos[i]
        assert np.all(g_sel[i, k:] == -1)
        a, b = set(ids.tolist()), set(o_sel[i, :k].tolist())
        if a == b:
            equal[i] = True
            continue
        t = scores[i, :pos[i] + 1]
        thr = GAP_REL * np.abs(t).max()
        boundary = t[o_sel[i, :k]].min()
        for x in a ^ b:
            assert abs(t[x] - boundary) < thr, f"query {i}: token {x} outside the near-tie band"
    return equal
