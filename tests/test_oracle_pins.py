"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values fixed
by construction (planted maxima), closed forms (uniform-weight attention,
p = 0), brute force over all candidate subsets, textbook library routines
(torch's scaled_dot_product_attention in fp64, scipy's Sylvester Hadamard,
numpy's IEEE fp16 conversion), exact integer arithmetic, and the properties
the pages state:
  * "Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support" (llama.cpp PR
    24908), Overview: the local block is always selected, top-16 blocks;
    review thread (RADV validation): below top_k * block = 2048 tokens every
    block is selected and MSA equals dense attention; k = min(top_k, nblk).
  * llama.cpp compare b10146, MSA commit log: prefill and decode rank the
    same scores, so they cannot disagree on selection.
  * "deepseek2 : GLM-DSA sparse attention (lightning indexer)" (ik_llama.cpp
    PR 2045): Hadamard-rotated F16 keys; top-k keys per query; at
    n_kv <= top_k the sparse mask is a no-op (dense equality).
Pure CPU; runs in a few seconds.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import workloads as W

SCALE = W.SCALE


# ---------------------------------------------------------------------------
# Storage-format conversions
# ---------------------------------------------------------------------------
def test_bf16_to_f64_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_to_f64(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f16_to_f64_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f64_to_f16_rne_against_ieee():
    rng = np.random.default_rng(1)
    finite = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = finite[np.isfinite(finite)].astype(np.float64)
    srt = np.sort(np.unique(finite))
    mids = (srt[:-1] + srt[1:]) / 2          # exact ties: must round to even
    xs = np.concatenate([
        finite, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
        rng.standard_normal(20000) * np.exp(rng.uniform(-20, 11, 20000)),
        [65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -24 * 1.5, 2.0 ** -26, 0.0, -0.0],
    ])
    ref = xs.astype(np.float16).view(np.uint16)
    got = oracle.f64_to_f16_bits(xs)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# MSA block scores: score -> causal mask -> 128-token max-pool
# ---------------------------------------------------------------------------
def _planted_stream(cap, rng):
    """idx_k whose score against idx_q = c_g * e_{d_g} is c_g * f[j, g]."""
    G, Di = W.N_GROUP, W.IDX_DIM
    d_g = np.array([5, 77, 31, 127])
    c_g = np.array([1.0, -2.0, 0.5, 4.0], np.float32)
    idx_k = rng.integers(-30, 31, size=(cap, G, Di)).astype(np.float32)   # noise off the planted dims
    f = rng.integers(-50, 51, size=(cap, G)).astype(np.float32)
    for g in range(G):
        idx_k[:, g, d_g[g]] = f[:, g]
    idx_q = np.zeros((1, G, Di), np.float32)
    for g in range(G):
        idx_q[0, g, d_g[g]] = c_g[g]
    return idx_k, idx_q, f, c_g


def test_block_scores_planted_max_and_causal_boundary():
    rng = np.random.default_rng(2)
    cap, p = 700, 600                      # ragged cache; local block 4 = slots 512..639
    idx_k, idx_q, f, c = _planted_stream(cap, rng)
    # plant: the query's own slot p carries block 4's max; slot p + 1 (not
    # visible) carries a larger value that must be ignored
    f[p, :] = 77.0
    f[p + 1, :] = 1000.0
    for g in range(4):
        idx_k[p, g, [5, 77, 31, 127][g]] = 77.0
        idx_k[p + 1, g, [5, 77, 31, 127][g]] = 1000.0
    bs, sel, n_sel = oracle.msa_select(idx_k[None], np.array([0]), np.array([p]), idx_q,
                                       nblk_out=6)
    for g in range(4):
        for b in range(5):
            hi = min((b + 1) * 128, p + 1)
            vals = c[g] * f[b * 128:hi, g].astype(np.float64)
            assert bs[0, g, b] == vals.max(), (g, b)
        assert bs[0, g, 5] == -np.inf
    # block 4 max for positive c_g is the planted self-slot value
    assert bs[0, 0, 4] == 77.0
    assert bs[0, 3, 4] == 4.0 * 77.0


def test_block_scores_brute_force_matmul_tiny():
    """Brute force through a dense fp64 product on a tiny ragged stream."""
    rng = np.random.default_rng(3)
    cap = 3 * 128 + 17
    idx_k = rng.standard_normal((2, cap, 4, 128)).astype(np.float32)
    idx_q = rng.standard_normal((5, 4, 128)).astype(np.float32)
    stream = np.array([0, 1, 1, 0, 1], np.int32)
    pos = np.array([0, 127, 128, 300, cap - 1], np.int32)
    bs, _, _ = oracle.msa_select(idx_k, stream, pos, idx_q, nblk_out=4)
    for i in range(5):
        for g in range(4):
            s = idx_k[stream[i], :, g, :].astype(np.float64) @ idx_q[i, g].astype(np.float64)
            s[np.arange(cap) > pos[i]] = -np.inf
            s = np.concatenate([s, np.full(4 * 128 - cap, -np.inf)]).reshape(4, 128).max(1)
            np.testing.assert_allclose(bs[i, g], s, rtol=1e-13, atol=1e-12)


def test_block_scores_exact_on_integer_inputs():
    """Integer-valued f32 inputs (the 1x4k workload's distribution): every
    score is an integer, so the fp64 result must equal exact int64 maths."""
    wl = W.decode_workload("t", 1, 1000, "int8")
    idx_k = W.stream_idx_k(wl, 0)
    idx_q = W.query_idx(wl, 0)
    bs, _, _ = oracle.msa_select(idx_k[None], np.array([0]), np.array([999]), idx_q[None],
                                 nblk_out=8)
    ki = idx_k.astype(np.int64)
    qi = idx_q.astype(np.int64)
    for g in range(4):
        s = ki[:, g, :] @ qi[g]
        for b in range(8):
            assert bs[0, g, b] == s[b * 128:min((b + 1) * 128, 1000)].max()


# ---------------------------------------------------------------------------
# Top-k selection
# ---------------------------------------------------------------------------
def _dominates(score, a, b):
    return score[a] > score[b] or (score[a] == score[b] and a < b)


def _brute_force_selection(score, local, top_k):
    """All subsets of size min(top_k, n) containing the local id whose every
    non-local member ranks above every non-member; must be exactly one."""
    n = len(score)
    k = min(top_k, n)
    others = [i for i in range(n) if i != local]
    found = []
    for comb in itertools.combinations(others, k - 1):
        chosen = set(comb)
        out = [u for u in others if u not in chosen]
        if all(_dominates(score, s, u) for s in chosen for u in out):
            found.append(sorted(chosen | {local}))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("n,top_k", [(1, 16), (5, 16), (9, 4), (12, 5), (18, 16), (17, 16)])
def test_selection_brute_force(n, top_k):
    rng = np.random.default_rng(100 + n * top_k)
    for trial in range(6):
        # small integer range: plenty of ties, which must go to the lower id
        score = rng.integers(-3, 4, size=n).astype(np.float64)
        local = int(rng.integers(0, n))
        got = oracle.select_ranked(score, local, top_k)
        want = _brute_force_selection(score, local, top_k)
        k = min(top_k, n)
        assert list(got[:k]) == want
        assert np.all(got[k:] == -1)


def test_selection_all_equal_scores():
    score = np.zeros(40)
    got = oracle.select_ranked(score, 33, 16)
    assert list(got) == list(range(15)) + [33]


def test_selection_invariants_large():
    """Local always in; count = min(16, nvis); ids <= local; every selected
    non-local block ranks above every unselected one."""
    wl = W.decode_workload("t", 3, 5000)
    ck = W.caches(wl)
    pos = np.array([0, 1919, 4999], np.int32)
    q = np.stack([W.query_idx(wl, i) for i in range(3)])
    bs, sel, n_sel = oracle.msa_select(ck["idx_k"], np.arange(3, dtype=np.int32), pos, q)
    for i in range(3):
        loc = pos[i] // 128
        for g in range(4):
            k = n_sel[i, g]
            assert k == min(16, loc + 1)
            s = sel[i, g, :k]
            assert np.all(np.diff(s) > 0) and np.all(sel[i, g, k:] == -1)
            assert loc in s and s.max() == loc
            chosen = [b for b in s if b != loc]
            rest = [b for b in range(loc + 1) if b not in s]
            sc = bs[i, g]
            for a in chosen:
                for b in rest:
                    assert _dominates(sc, a, b)


def test_prefill_equals_per_query_decode():
    """Unified selection: a chunk of consecutive queries selects exactly what
    each query selects alone."""
    wl = W.prefill_workload("t", 2000, 1500, 40)
    ck = W.caches(wl)
    qs = W.queries(wl)
    _, sel_all, _ = oracle.msa_select(ck["idx_k"], qs["stream"], qs["pos"], qs["idx_q"])
    for i in range(0, 40, 7):
        _, sel_one, _ = oracle.msa_select(ck["idx_k"], qs["stream"][i:i + 1], qs["pos"][i:i + 1],
                                          qs["idx_q"][i:i + 1])
        assert np.array_equal(sel_one[0], sel_all[i])


# ---------------------------------------------------------------------------
# Sparse attention
# ---------------------------------------------------------------------------
def _bf16_to_torch64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def _dense_sdpa(k_s, v_s, q_i, p, mask_tokens=None):
    """Textbook attention of one query over keys 0..p (optionally restricted
    to a token mask) via torch's fp64 scaled_dot_product_attention."""
    G, Hg = W.N_GROUP, W.HEADS_PER_GROUP
    k = _bf16_to_torch64(k_s[:p + 1])                 # [p+1][G][D]
    v = _bf16_to_torch64(v_s[:p + 1])
    q = _bf16_to_torch64(q_i)                         # [H][D]
    kh = k.permute(1, 0, 2).repeat_interleave(Hg, 0)  # [H][p+1][D]
    vh = v.permute(1, 0, 2).repeat_interleave(Hg, 0)
    mask = None
    if mask_tokens is not None:
        mask = torch.from_numpy(mask_tokens[:, :p + 1]).repeat_interleave(Hg, 0)[:, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], kh, vh, attn_mask=mask, scale=SCALE)
    return out[:, 0, :].numpy()


def test_attention_equals_dense_below_2048_tokens():
    wl = W.decode_workload("t", 2, 2048)
    ck = W.caches(wl)
    pos = np.array([2047, 777], np.int32)
    stream = np.array([0, 1], np.int32)
    qs = W.queries(wl)
    _, sel, n_sel = oracle.msa_select(ck["idx_k"], stream, pos, qs["idx_q"])
    assert n_sel[0].tolist() == [16] * 4 and n_sel[1].tolist() == [7] * 4
    out = oracle.sparse_attend(ck["k"], ck["v"], stream, pos, qs["q"], sel, unit=128, scale=SCALE)
    for i in range(2):
        ref = _dense_sdpa(ck["k"][stream[i]], ck["v"][stream[i]], qs["q"][i], pos[i])
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)


def test_attention_equals_masked_dense_at_long_context():
    """Above 2048 tokens: the sparse result equals dense attention restricted
    by an explicit token mask of the selected blocks (partial local block)."""
    wl = W.decode_workload("t", 1, 5000)
    ck = W.caches(wl)
    qs = W.queries(wl)
    pos = np.array([4321], np.int32)
    _, sel, _ = oracle.msa_select(ck["idx_k"], np.array([0], np.int32), pos, qs["idx_q"])
    out = oracle.sparse_attend(ck["k"], ck["v"], np.array([0], np.int32), pos, qs["q"], sel,
                               unit=128, scale=SCALE)
    mask = np.zeros((4, 5000), bool)
    for g in range(4):
        for b in sel[0, g]:
            mask[g, b * 128:(b + 1) * 128] = True
    ref = _dense_sdpa(ck["k"][0], ck["v"][0], qs["q"][0], 4321, mask_tokens=mask)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def test_attention_zero_query_is_mean_of_selected_values():
    wl = W.decode_workload("t", 1, 3000)
    ck = W.caches(wl)
    pos = np.array([2999], np.int32)
    sel = np.full((1, 4, 16), -1, np.int32)
    sel[0, :, :3] = [[0, 9, 23], [4, 5, 23], [1, 2, 23], [7, 8, 23]]
    q = np.zeros((1, 64, 128), np.uint16)              # +0.0 in bf16
    out = oracle.sparse_attend(ck["k"], ck["v"], np.array([0], np.int32), pos, q, sel,
                               unit=128, scale=SCALE)
    vv = oracle.bf16_to_f64(ck["v"][0].reshape(-1)).reshape(3000, 4, 128)
    for g in range(4):
        toks = [j for b in sel[0, g] if b >= 0 for j in range(b * 128, (b + 1) * 128) if j <= 2999]
        mean = vv[toks, g, :].mean(0)
        for h in range(16):
            np.testing.assert_allclose(out[0, g * 16 + h], mean, rtol=1e-13, atol=1e-14)


def test_attention_at_position_zero_returns_first_value():
    wl = W.decode_workload("t", 1, 256)
    ck = W.caches(wl)
    qs = W.queries(wl)
    pos = np.array([0], np.int32)
    _, sel, n_sel = oracle.msa_select(ck["idx_k"], np.array([0], np.int32), pos, qs["idx_q"][:1])
    assert n_sel.tolist() == [[1, 1, 1, 1]]
    out = oracle.sparse_attend(ck["k"], ck["v"], np.array([0], np.int32), pos, qs["q"][:1], sel,
                               unit=128, scale=SCALE)
    v0 = oracle.bf16_to_f64(ck["v"][0, 0].reshape(-1)).reshape(4, 128)
    for h in range(64):
        assert np.array_equal(out[0, h], v0[h // 16])


def test_attention_one_hot_values_give_block_weights():
    """V[j] = e_{block(j)}: output column b is the softmax mass on block b; it
    is zero outside the selected blocks and sums to one."""
    wl = W.decode_workload("t", 1, 40 * 128)
    ck = W.caches(wl)
    qs = W.queries(wl)
    pos = np.array([40 * 128 - 50], np.int32)
    _, sel, _ = oracle.msa_select(ck["idx_k"], np.array([0], np.int32), pos, qs["idx_q"])
    v = np.zeros_like(ck["v"])
    blocks = np.arange(40 * 128) // 128
    v[0, np.arange(40 * 128), :, blocks] = 0x3F80     # bf16 1.0
    out = oracle.sparse_attend(ck["k"], v, np.array([0], np.int32), pos, qs["q"], sel,
                               unit=128, scale=SCALE)
    for h in range(64):
        g = h // 16
        mass = out[0, h, :40]
        unselected = np.setdiff1d(np.arange(40), sel[0, g])
        assert np.all(mass[unselected] == 0.0)
        assert np.all(mass[sel[0, g]] > 0.0)
        assert abs(mass.sum() - 1.0) < 1e-13
        assert np.all(out[0, h, 40:] == 0.0)


# ---------------------------------------------------------------------------
# DSA lightning indexer
# ---------------------------------------------------------------------------
def test_dsa_rotation_of_unit_vectors_is_sylvester_hadamard():
    n = 128
    eye = np.zeros((n, n), np.uint16)
    eye[np.arange(n), np.arange(n)] = 0x3C00            # fp16 1.0
    cols = oracle.dsa_rotate(eye)                       # row i = H e_i / sqrt(n)
    ref = (scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)).T.astype(np.float16).view(np.uint16)
    assert np.array_equal(cols, ref)
    signs = np.where(cols.view(np.float16) > 0, 1, -1)
    assert np.array_equal(signs @ signs.T, n * np.eye(n, dtype=int))   # H H^T = n I


def test_dsa_rotation_matches_library_hadamard_product():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)).astype(np.float16)
    got = oracle.dsa_rotate(x.view(np.uint16))
    H = scipy.linalg.hadamard(128).astype(np.float64)
    ref = ((x.astype(np.float64) @ H.T) * (1.0 / math.sqrt(128))).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_dsa_topk_equals_full_sort_with_ties():
    rng = np.random.default_rng(6)
    cap = 300
    k_rot = rng.integers(-2, 3, size=(1, cap, 128)).astype(np.float16).view(np.uint16)
    q = rng.integers(-1, 2, size=(3, 128)).astype(np.float16).view(np.uint16)
    pos = np.array([299, 150, 40], np.int32)
    sel, n_sel, scores = oracle.dsa_select(k_rot, np.zeros(3, np.int32), pos, q, top_k=64,
                                           want_scores=True)
    kk = k_rot.view(np.float16).astype(np.int64)[0]
    for i in range(3):
        s = kk[:pos[i] + 1] @ q[i].view(np.float16).astype(np.int64)
        order = np.lexsort((np.arange(pos[i] + 1), -s))    # score desc, id asc
        want = np.sort(order[:min(64, pos[i] + 1)])
        assert n_sel[i] == min(64, pos[i] + 1)
        assert np.array_equal(sel[i, :n_sel[i]], want)
        assert np.all(sel[i, n_sel[i]:] == -1)
        assert np.array_equal(scores[i, :pos[i] + 1], s.astype(np.float64))


def test_dsa_short_context_is_dense_attention():
    """n_kv <= top_k: every token kept, the result is dense attention."""
    wl = W.decode_workload("t", 1, 1500, kind="dsa_decode")
    ck = W.caches(wl)
    qs = W.queries(wl)
    k_rot = oracle.dsa_rotate(ck["dsa_k"])
    pos = np.array([1499], np.int32)
    sel, n_sel, _ = oracle.dsa_select(k_rot, np.array([0], np.int32), pos, qs["q_idx"][:1])
    assert n_sel[0] == 1500 and np.array_equal(sel[0, :1500], np.arange(1500))
    out = oracle.sparse_attend(ck["k"], ck["v"], np.array([0], np.int32), pos, qs["q"][:1], sel,
                               unit=1, scale=SCALE, shared_across_groups=True)
    ref = _dense_sdpa(ck["k"][0], ck["v"][0], qs["q"][0], 1499)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def _f16(a):
    return np.asarray(a, np.float16).view(np.uint16)


def test_dsa_heads_hand_worked_example():
    """Two heads, 2-dim keys, worked by hand:
    q0 = (2, 1), q1 = (-1, 3), w = (1, 0.5);
    k0 = (1, 0): max(0, 2) + 0.5 max(0, -1) = 2
    k1 = (0, 1): 1 + 0.5 * 3 = 2.5
    k2 = (1, 1): 3 + 0.5 * 2 = 4
    k3 = (-1, 2): max(0, -1) + 0.5 * 7 = 3.5"""
    k = _f16([[[1, 0], [0, 1], [1, 1], [-1, 2]]])
    q = _f16([[[2, 1], [-1, 3]]])
    w = np.array([[1.0, 0.5]], np.float32)
    sel, n_sel, sc = oracle.dsa_select_heads(k, [0], [3], q, w, top_k=2, want_scores=True)
    assert np.array_equal(sc[0], [2.0, 2.5, 4.0, 3.5])
    assert n_sel[0] == 2 and np.array_equal(sel[0], [2, 3])
    sel, n_sel, _ = oracle.dsa_select_heads(k, [0], [1], q, w, top_k=2)   # causal: keys 0, 1 only
    assert n_sel[0] == 2 and np.array_equal(sel[0], [0, 1])


def test_dsa_heads_brute_force_exact():
    """Small integers and dyadic weights: every sum is exact, so the oracle
    must equal a rational-arithmetic evaluation of the formula."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    H, D, cap, n_q = 3, 8, 12, 4
    k = rng.integers(-3, 4, size=(2, cap, D))
    q = rng.integers(-3, 4, size=(n_q, H, D))
    w = rng.integers(-4, 5, size=(n_q, H)) / 4.0
    stream = np.array([0, 1, 1, 0], np.int32)
    pos = np.array([11, 5, 0, 7], np.int32)
    sel, n_sel, sc = oracle.dsa_select_heads(_f16(k), stream, pos, _f16(q), w.astype(np.float32), top_k=5,
                                             want_scores=True)
    for i in range(n_q):
        want = []
        for j in range(pos[i] + 1):
            tot = Fraction(0)
            for h in range(H):
                dot = sum(int(q[i, h, d]) * int(k[stream[i], j, d]) for d in range(D))
                tot += Fraction(w[i, h]) * max(0, dot)
            want.append(tot)
        assert [Fraction(x) for x in sc[i, :pos[i] + 1]] == want
        assert np.all(np.isneginf(sc[i, pos[i] + 1:]))
        order = sorted(range(pos[i] + 1), key=lambda j: (-want[j], j))
        kk = min(5, pos[i] + 1)
        assert n_sel[i] == kk and list(sel[i, :kk]) == sorted(order[:kk])
        assert np.all(sel[i, kk:] == -1)


def test_dsa_heads_single_positive_head_is_single_head_select():
    """One head of weight 1 whose dot products are all positive is the
    single-head indexer."""
    rng = np.random.default_rng(12)
    k = _f16(rng.uniform(0.1, 1.0, size=(2, 400, 128)))
    q = _f16(rng.uniform(0.1, 1.0, size=(3, 128)))
    stream, pos = np.array([0, 1, 1], np.int32), np.array([399, 200, 37], np.int32)
    s1, n1, sc1 = oracle.dsa_select(k, stream, pos, q, top_k=64, want_scores=True)
    s2, n2, sc2 = oracle.dsa_select_heads(k, stream, pos, q[:, None, :], np.ones((3, 1), np.float32),
                                          top_k=64, want_scores=True)
    assert np.array_equal(sc1, sc2) and np.array_equal(s1, s2) and np.array_equal(n1, n2)


def test_dsa_heads_relu_sign_and_linearity():
    rng = np.random.default_rng(13)
    H, D, cap = 4, 16, 64
    k = rng.integers(-2, 3, size=(1, cap, D))
    q = rng.integers(-2, 3, size=(2, H, D))
    w = (rng.integers(-4, 5, size=(2, H)) / 8.0).astype(np.float32)
    pos = np.array([63, 40], np.int32)
    st = np.zeros(2, np.int32)
    score = lambda qq, ww: oracle.dsa_select_heads(_f16(k), st, pos, _f16(qq), ww, top_k=8, want_scores=True)[2]
    base = score(q, w)
    # a head with no positive dot product adds nothing, whatever its weight
    kpos = np.abs(k)
    kpos[..., 0] += 1                                   # every key has a positive first entry
    qneg = np.concatenate([q, -np.ones((2, 1, D), np.int64)], axis=1)
    for wx in (-3.0, 0.0, 5.0):
        w5 = np.concatenate([w, np.full((2, 1), wx, np.float32)], axis=1)
        a = oracle.dsa_select_heads(_f16(kpos), st, pos, _f16(qneg), w5, top_k=8, want_scores=True)[2]
        b = oracle.dsa_select_heads(_f16(kpos), st, pos, _f16(q), w, top_k=8, want_scores=True)[2]
        assert np.array_equal(a, b)
    # the ReLU acts per head before the weights: negating a query head is not
    # negating its contribution
    fin = np.isfinite(base)
    assert not np.array_equal(score(-q, w)[fin], -base[fin])
    # linear in the weights, and odd in them
    w2 = (rng.integers(-4, 5, size=(2, H)) / 8.0).astype(np.float32)
    assert np.array_equal(score(q, w + w2)[fin], base[fin] + score(q, w2)[fin])
    assert np.array_equal(score(q, -w)[fin], -base[fin])


def test_index_project_hand_worked():
    """x = (1, 2), W = [[1, 1], [1, -1]]: y = (3, -1), rms = sqrt(5).
    pos 0: z = (3, -1) / sqrt(5) * (1 + gamma) with gamma = (0, 0.5);
    pos 1 (rot_dim 2, one pair, frequency theta^0 = 1): rotate by 1 rad."""
    x = np.array([[1.0, 2.0], [1.0, 2.0]], np.float32)
    w = np.array([[1, 1], [1, -1]], np.float32)
    g = np.array([[0.0, 0.5]], np.float32)
    q, _ = oracle.index_project(x, w, w, g, g, [0, 1], eps=0.0, theta=10000.0, rot_dim=2, n_group=1,
                                want_k=False)
    a, b = 3 / math.sqrt(5), -1.5 / math.sqrt(5)
    np.testing.assert_allclose(q[0, 0], [a, b], rtol=1e-15)
    np.testing.assert_allclose(q[1, 0], [a * math.cos(1) - b * math.sin(1), a * math.sin(1) + b * math.cos(1)],
                               rtol=1e-14)


def _proj_inputs(seed, n_tok=5, d=96, hd=128, n_group=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_tok, d)).astype(np.float32)
    w = (rng.standard_normal((n_group * hd, d)) / math.sqrt(d)).astype(np.float32)
    g = (0.1 * rng.standard_normal((n_group, hd))).astype(np.float32)
    return x, w, g


def test_index_project_rope_angles():
    """y = c * e_i for one i at a time: the rotated pair (i, i + 32) must make
    the angle pos * theta^(-2 i / 64) with the first axis."""
    hd, rot, theta = 128, 64, 10000.0
    for i in (0, 1, 7, 31):
        w = np.zeros((hd, 1), np.float32)
        w[i, 0] = 1.0
        for p in (1, 5, 1000, 32767):
            q, _ = oracle.index_project(np.ones((1, 1), np.float32), w, w, np.zeros((1, hd), np.float32),
                                        np.zeros((1, hd), np.float32), [p], eps=0.0, theta=theta, rot_dim=rot,
                                        n_group=1, want_k=False)
            ang = p * theta ** (-2.0 * i / rot)
            z = math.sqrt(hd)                                  # e_i normalised to rms 1
            np.testing.assert_allclose([q[0, 0, i], q[0, 0, i + rot // 2]], [z * math.cos(ang), z * math.sin(ang)],
                                       rtol=1e-12, atol=1e-12)
            others = np.delete(q[0, 0], [i, i + rot // 2])
            assert np.all(others == 0.0)


def test_index_project_relative_position():
    """RoPE: q at a and k at b score the same as q at a + c and k at b + c."""
    x, w, g = _proj_inputs(21, n_tok=1)
    xs = np.repeat(x, 4, axis=0)
    q, k = oracle.index_project(xs, w, w[::-1].copy(), g, g[::-1].copy(), [100, 37, 30100, 30037],
                                eps=1e-6, theta=10000.0, rot_dim=64)
    for gg in range(4):
        assert abs(q[0, gg] @ k[1, gg] - q[2, gg] @ k[3, gg]) < 1e-9 * np.abs(q[0, gg]).sum() * np.abs(k[1, gg]).max()
    assert abs(q[0, 0] @ k[1, 0] - q[0, 0] @ k[3, 0]) > 1e-6      # not position-independent


def test_index_project_norm_and_library_reduction():
    x, w, g = _proj_inputs(22)
    z = np.zeros_like(g)
    pos = np.array([0, 3, 100, 4095, 32767], np.int32)
    q0, _ = oracle.index_project(x, w, w, z, z, np.zeros(5, np.int32), eps=0.0, theta=10000.0, rot_dim=64,
                                 want_k=False)
    y = (x.astype(np.float64) @ w.astype(np.float64).T).reshape(5, 4, 128)
    ref = y / np.sqrt((y ** 2).mean(-1, keepdims=True))
    np.testing.assert_allclose(q0, ref, rtol=1e-12, atol=1e-12)
    # eps: the mean square is mean(y^2) / (mean(y^2) + eps)
    eps = 0.25
    qe, _ = oracle.index_project(x, w, w, z, z, np.zeros(5, np.int32), eps=eps, theta=10000.0, rot_dim=64,
                                 want_k=False)
    ms = (y ** 2).mean(-1)
    np.testing.assert_allclose((qe ** 2).mean(-1), ms / (ms + eps), rtol=1e-12)
    # RoPE keeps each head's norm and leaves dims >= 64 unchanged
    qp, _ = oracle.index_project(x, w, w, g, g, pos, eps=1e-6, theta=10000.0, rot_dim=64, want_k=False)
    qg, _ = oracle.index_project(x, w, w, g, g, np.zeros(5, np.int32), eps=1e-6, theta=10000.0, rot_dim=64,
                                 want_k=False)
    np.testing.assert_allclose(np.linalg.norm(qp, axis=-1), np.linalg.norm(qg, axis=-1), rtol=1e-12)
    assert np.array_equal(qp[..., 64:], qg[..., 64:])
    assert not np.allclose(qp[1:, :, :64], qg[1:, :, :64])


def _bf16_bits(x):
    return W.to_bf16_bits(np.asarray(x, np.float32))


@pytest.mark.parametrize("fmt,qmax", [(1, 127), (2, 7)])
def test_kv_quantize_round_trip_and_exact_grid(fmt, qmax):
    rng = np.random.default_rng(31)
    x = _bf16_bits(rng.standard_normal((50, 128)))
    codes, sc = oracle.kv_quantize(x, fmt)
    xf = x.astype(np.uint32) << 16
    xv = xf.view(np.float32).astype(np.float64)
    deq = oracle.kv_dequantize(codes, sc, fmt)
    # within half a step of the original, step = amax / qmax per 32 values; the f32
    # quotient x / s carries up to 2^-24 * qmax of error, so a value next to a
    # half step may round to the farther code (relative excess <= 2 * 2^-24 * qmax)
    step = np.repeat(sc.astype(np.float64), 32, axis=-1)
    assert np.all(np.abs(deq - xv) <= 0.5 * step * (1 + 2e-5))
    np.testing.assert_array_equal(sc, (np.abs(xv).reshape(50, 4, 32).max(-1) / qmax).astype(np.float32))
    # values on the exact grid c * 2^-3 with amax = qmax * 2^-3: codes exact, round trip exact
    c = rng.integers(-qmax, qmax + 1, size=(3, 128))
    c[:, ::32] = qmax
    grid = c * 0.125
    codes, sc = oracle.kv_quantize(_bf16_bits(grid), fmt)
    assert np.all(sc == 0.125)
    np.testing.assert_array_equal(oracle.kv_dequantize(codes, sc, fmt), grid)
    # an all-zero block gives scale 0 and zero codes
    z = np.zeros((1, 128), np.uint16)
    codes, sc = oracle.kv_quantize(z, fmt)
    assert np.all(sc == 0) and np.all(oracle.kv_dequantize(codes, sc, fmt) == 0)


def test_kv_q4_nibble_layout():
    """One 32-value block on the integer grid, codes c_j = (j % 15) - 7 (amax 7,
    so the scale is 1): byte j holds c_j + 8 (low nibble) and c_{j+16} + 8 (high)."""
    c = np.array([(j % 15) - 7 for j in range(32)], np.int64)
    c[1] = 7
    codes, sc = oracle.kv_quantize(_bf16_bits(c[None, :].astype(np.float32)), 2)
    assert sc[0, 0] == 1.0
    for j in range(16):
        assert codes[0, j] == (c[j] + 8) | ((c[j + 16] + 8) << 4)


def test_attend_f64_equals_bf16_attention_on_bf16_values():
    wl = W.Workload("t", "msa_decode", 2, 600, (0, 1, 1), (599, 300, 5))
    ck = W.caches(wl)
    qs = W.queries(wl)
    sel = np.full((3, 4, 16), -1, np.int32)
    for i, p in enumerate(qs["pos"]):
        nb = p // 128 + 1
        sel[i, :, :nb] = np.arange(nb)
    a = oracle.sparse_attend(ck["k"], ck["v"], qs["stream"], qs["pos"], qs["q"], sel, unit=128, scale=W.SCALE)
    to64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    b = oracle.sparse_attend_f64(to64(ck["k"]), to64(ck["v"]), qs["stream"], qs["pos"], qs["q"], sel, unit=128,
                                 scale=W.SCALE)
    assert np.array_equal(a, b)


def _read_golden_1x4k():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "decode_1x4k_int.txt")
    bs, sel = {}, {}
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        tag, g, *vals = line.split()
        (bs if tag == "bs" else sel)[int(g)] = [int(v) for v in vals]
    return bs, sel


def test_golden_1x4k_integer_fixture():
    """The stored integer block maxima equal exact int64 maths on the seeded
    inputs, and the oracle still reproduces the stored selection."""
    wl = W.CONFIGS["decode_1x4k_int"]
    gbs, gsel = _read_golden_1x4k()
    idx_k = W.stream_idx_k(wl, 0).astype(np.int64)
    idx_q = W.query_idx(wl, 0).astype(np.int64)
    for g in range(4):
        s = idx_k[:, g, :] @ idx_q[g]
        assert gbs[g] == [int(x) for x in s.reshape(32, 128).max(1)]
    ck = W.caches(wl)
    qs = W.queries(wl)
    bs, sel, _ = oracle.msa_select(ck["idx_k"], qs["stream"], qs["pos"], qs["idx_q"])
    for g in range(4):
        assert [int(x) for x in bs[0, g]] == gbs[g]
        assert sel[0, g].tolist() == gsel[g]
