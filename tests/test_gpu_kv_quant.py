"""GPU parity of quantized K/V caches (msa_cache.kv_format: int8, or 4-bit
codes, one f32 scale per 32 values) against the fp64 oracle, through the C ABI.

* Append: codes and scales bit-exact against the oracle's quantizer (the
  decisions are taken in f32 on both sides).
* Decode attention (MSA blocks and DSA token ids): against fp64 attention on
  the oracle's dequantized caches, to the attention tolerances (the kernel
  multiplies exact codes: K's scales scale each 32-dim slice of the scores, V's
  are folded into the bf16 probabilities, the one rounding, as in the bf16
  path), for splits of 2, 4 and 8 units.
* Prefill attention (msa_attend_prefill) on quantized caches: the tile sweep
  over a bf16 copy of the used blocks, each dequantized value rounded once to
  bf16; the same tolerances against fp64 attention on the dequantized caches.
* Paged quantized caches: bit-identical to per-stream ones.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import oracle
import workloads as W
from _gpu_common import DEV, check_attention, dev, dev_bits, log

pytestmark = pytest.mark.gpu

FMTS = [(M.KV_INT8, "int8"), (M.KV_Q4, "q4")]


def _alloc(S, cap, fmt):
    width = 128 if fmt == M.KV_INT8 else 64
    k = torch.zeros((S, cap, 4, width), dtype=torch.uint8, device=DEV)
    v = torch.zeros_like(k)
    ks = torch.zeros((S, cap, 4, 4), dtype=torch.float32, device=DEV)
    vs = torch.zeros_like(ks)
    return k, v, ks, vs


def _append_all(cache, host, S, cap, dims, dsa=False):
    """Append every (stream, position) row through the entry point."""
    st = torch.arange(S, dtype=torch.int32, device=DEV).repeat_interleave(cap)
    ps = torch.arange(cap, dtype=torch.int32, device=DEV).repeat(S)
    kn = dev_bits(host["k"].reshape(S * cap, 4, 128), torch.bfloat16)
    vn = dev_bits(host["v"].reshape(S * cap, 4, 128), torch.bfloat16)
    if dsa:
        M.dsa_index_append(dims, cache, st, ps, cap - 1, dev_bits(host["dsa_k"].reshape(S * cap, 128), torch.float16),
                           kn, vn)
    else:
        M.msa_index_append(dims, cache, st, ps, cap - 1, dev(host["idx_k"].reshape(S * cap, 4, 128)), kn, vn)
    torch.cuda.synchronize()


def _oracle_caches(host, fmt):
    kc, ksc = oracle.kv_quantize(host["k"], fmt)
    vc, vsc = oracle.kv_quantize(host["v"], fmt)
    return (kc, ksc, vc, vsc), oracle.kv_dequantize(kc, ksc, fmt), oracle.kv_dequantize(vc, vsc, fmt)


@pytest.mark.parametrize("fmt,name", FMTS)
def test_kv_quant_msa_decode(fmt, name):
    pos = (0, 1, 127, 128, 129, 1000, 2047, 2048, 2049, 3999, 2500, 777)
    wl = W.Workload(f"kvq_{name}", "msa_decode", 3, 4000, tuple(i % 3 for i in range(len(pos))), pos)
    log(f"[kv quant {name}] msa decode: streams={wl.n_stream} cap={wl.cap} n_q={wl.n_q}")
    host, qs = W.caches(wl), W.queries(wl)
    S, cap = wl.n_stream, wl.cap
    k, v, ks, vs = _alloc(S, cap, fmt)
    idx = torch.zeros((S, cap, 4, 128), dtype=torch.float32, device=DEV)
    dims = M.msa_dims(wl.top_k, W.SCALE)
    cache = M.make_cache(k=k, v=v, idx_k=idx, kv_format=fmt, k_scale=ks, v_scale=vs)
    _append_all(cache, host, S, cap, dims)
    (kc, ksc, vc, vsc), kd, vd = _oracle_caches(host, fmt)
    assert np.array_equal(k.cpu().numpy(), kc) and np.array_equal(v.cpu().numpy(), vc), "codes differ"
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), ksc.view(np.uint32)), "k scales differ"
    assert np.array_equal(vs.cpu().numpy().view(np.uint32), vsc.view(np.uint32)), "v scales differ"
    _, o_sel, _ = oracle.msa_select(host["idx_k"], qs["stream"], qs["pos"], qs["idx_q"])
    out = torch.empty((wl.n_q, 64, 128), device=DEV)
    ws = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_ATTEND_DECODE, wl.n_q, wl.max_pos), 256),
                     dtype=torch.uint8, device=DEV)
    M.msa_attend_decode(dims, cache, dev_bits(qs["q"], torch.bfloat16), dev(qs["stream"]), dev(qs["pos"]),
                        wl.max_pos, dev(o_sel), out, ws)
    torch.cuda.synchronize()
    ref = oracle.sparse_attend_f64(kd, vd, qs["stream"], qs["pos"], qs["q"], o_sel, unit=128, scale=W.SCALE)
    wa, wr = check_attention(out.cpu().numpy(), ref)
    log(f"  codes and scales bit-exact; attention max-abs {wa:.3e}, rel-L2 {wr:.3e}")


@pytest.mark.parametrize("fmt,name", FMTS)
@pytest.mark.parametrize("cap,pos0,n_q", [(3000, 1900, 300), (6000, 5000, 200)])
def test_kv_quant_msa_prefill(fmt, name, cap, pos0, n_q):
    """Prefill chunks of 300 consecutive queries (nine full 32-query tiles and a
    ragged 12; selections holding most of the ~17 visible blocks) and of 200
    (16 of ~40 blocks) over quantized caches whose capacity is not a multiple
    of 128."""
    wl = W.prefill_workload(f"kvq_pf_{name}_{pos0}", cap, pos0, n_q)
    log(f"[kv quant {name}] msa prefill: cap={wl.cap} pos0={wl.pos[0]} n_q={wl.n_q}")
    host, qs = W.caches(wl), W.queries(wl)
    S, cap = wl.n_stream, wl.cap
    k, v, ks, vs = _alloc(S, cap, fmt)
    idx = torch.zeros((S, cap, 4, 128), dtype=torch.float32, device=DEV)
    dims = M.msa_dims(wl.top_k, W.SCALE)
    cache = M.make_cache(k=k, v=v, idx_k=idx, kv_format=fmt, k_scale=ks, v_scale=vs)
    _append_all(cache, host, S, cap, dims)
    _, kd, vd = _oracle_caches(host, fmt)
    _, o_sel, _ = oracle.msa_select(host["idx_k"], qs["stream"], qs["pos"], qs["idx_q"])
    q = dev_bits(qs["q"], torch.bfloat16)
    out = torch.empty((wl.n_q, 64, 128), device=DEV)
    ws = torch.empty(M.workspace_bytes(dims, M.MSA_OP_ATTEND_PREFILL, wl.n_q, wl.max_pos), dtype=torch.uint8,
                     device=DEV)
    M.msa_attend_prefill(dims, cache, q, wl.stream[0], wl.pos[0], dev(o_sel), out, ws)
    torch.cuda.synchronize()
    ref = oracle.sparse_attend_f64(kd, vd, qs["stream"], qs["pos"], qs["q"], o_sel, unit=128, scale=W.SCALE)
    wa, wr = check_attention(out.cpu().numpy(), ref)
    log(f"  attention max-abs {wa:.3e}, rel-L2 {wr:.3e}")


@pytest.mark.parametrize("fmt,name", FMTS)
def test_kv_quant_msa_decode_eight_units_per_split(fmt, name):
    """32 queries x 16 selected blocks: two splits of eight units each, the
    kernel instance the 32 x 32K decode step runs."""
    S, cap = 32, 4096
    wl = W.Workload(f"kvq8_{name}", "msa_decode", S, cap, tuple(range(S)), tuple([cap - 1] * 16 + [2500] * 16))
    log(f"[kv quant {name}] 32 queries, 8 units per split")
    host, qs = W.caches(wl), W.queries(wl)
    k, v, ks, vs = _alloc(S, cap, fmt)
    idx = torch.zeros((S, cap, 4, 128), dtype=torch.float32, device=DEV)
    dims = M.msa_dims(wl.top_k, W.SCALE)
    cache = M.make_cache(k=k, v=v, idx_k=idx, kv_format=fmt, k_scale=ks, v_scale=vs)
    _append_all(cache, host, S, cap, dims)
    _, kd, vd = _oracle_caches(host, fmt)
    _, o_sel, _ = oracle.msa_select(host["idx_k"], qs["stream"], qs["pos"], qs["idx_q"])
    out = torch.empty((wl.n_q, 64, 128), device=DEV)
    ws = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_ATTEND_DECODE, wl.n_q, wl.max_pos), 256),
                     dtype=torch.uint8, device=DEV)
    M.msa_attend_decode(dims, cache, dev_bits(qs["q"], torch.bfloat16), dev(qs["stream"]), dev(qs["pos"]),
                        wl.max_pos, dev(o_sel), out, ws)
    torch.cuda.synchronize()
    ref = oracle.sparse_attend_f64(kd, vd, qs["stream"], qs["pos"], qs["q"], o_sel, unit=128, scale=W.SCALE)
    wa, wr = check_attention(out.cpu().numpy(), ref)
    log(f"  attention max-abs {wa:.3e}, rel-L2 {wr:.3e}")


@pytest.mark.parametrize("fmt,name", FMTS)
def test_kv_quant_dsa_decode(fmt, name):
    wl = W.Workload(f"kvq_dsa_{name}", "dsa_decode", 2, 3000, (0, 1, 0), (2999, 1500, 700), top_k=512)
    log(f"[kv quant {name}] dsa decode")
    host, qs = W.caches(wl), W.queries(wl)
    S, cap = wl.n_stream, wl.cap
    k, v, ks, vs = _alloc(S, cap, fmt)
    dsa_k = torch.zeros((S, cap, 128), dtype=torch.float16, device=DEV)
    dims = M.dsa_dims(wl.top_k, W.SCALE)
    cache = M.make_cache(k=k, v=v, dsa_k=dsa_k, kv_format=fmt, k_scale=ks, v_scale=vs)
    _append_all(cache, host, S, cap, dims, dsa=True)
    _, kd, vd = _oracle_caches(host, fmt)
    o_sel, _, _ = oracle.dsa_select(oracle.dsa_rotate(host["dsa_k"]), qs["stream"], qs["pos"], qs["q_idx"],
                                    top_k=wl.top_k)
    out = torch.empty((wl.n_q, 64, 128), device=DEV)
    ws = torch.empty(max(M.workspace_bytes(dims, M.DSA_OP_ATTEND_DECODE, wl.n_q, wl.max_pos), 256),
                     dtype=torch.uint8, device=DEV)
    M.dsa_attend_decode(dims, cache, dev_bits(qs["q"], torch.bfloat16), dev(qs["stream"]), dev(qs["pos"]),
                        wl.max_pos, dev(o_sel), out, ws)
    torch.cuda.synchronize()
    ref = oracle.sparse_attend_f64(kd, vd, qs["stream"], qs["pos"], qs["q"], o_sel, unit=1, scale=W.SCALE,
                                   shared_across_groups=True)
    wa, wr = check_attention(out.cpu().numpy(), ref)
    log(f"  attention max-abs {wa:.3e}, rel-L2 {wr:.3e}")


def test_kv_quant_paged_equals_per_stream():
    """Decode and prefill attention over a paged int8 cache (blocks placed by a
    random table) are bit-identical to those over per-stream caches."""
    fmt = M.KV_INT8
    wl = W.Workload("kvq_paged", "msa_decode", 2, 3000, (0, 1, 1), (2999, 2000, 128))
    log("[kv quant] paged vs per-stream")
    host, qs = W.caches(wl), W.queries(wl)
    S, cap = wl.n_stream, wl.cap
    nb = (cap + 127) // 128
    rng = np.random.default_rng(5)
    table = rng.permutation(S * nb + 2)[: S * nb].astype(np.int32).reshape(S, nb)
    n_pages = S * nb + 2
    dims = M.msa_dims(wl.top_k, W.SCALE)
    _, o_sel, _ = oracle.msa_select(host["idx_k"], qs["stream"], qs["pos"], qs["idx_q"])
    pwl = W.prefill_workload("kvq_paged_pf", cap, 1700, 300, stream=1, n_stream=S)
    pqs = W.queries(pwl)
    _, p_sel, _ = oracle.msa_select(host["idx_k"], pqs["stream"], pqs["pos"], pqs["idx_q"])
    pre_q = {paged: {"q": dev_bits(pqs["q"], torch.bfloat16), "sel": dev(p_sel),
                     "out": torch.empty((300, 64, 128), device=DEV)} for paged in (False, True)}
    outs = []
    for paged in (False, True):
        if paged:
            k = torch.zeros((n_pages * 128, 4, 128), dtype=torch.uint8, device=DEV)
            v = torch.zeros_like(k)
            ks = torch.zeros((n_pages * 128, 4, 4), dtype=torch.float32, device=DEV)
            vs = torch.zeros_like(ks)
            idx = torch.zeros((n_pages * 128, 4, 128), dtype=torch.float32, device=DEV)
            cache = M.make_cache(k=k, v=v, idx_k=idx, kv_format=fmt, k_scale=ks, v_scale=vs,
                                 block_table=dev(table), cap=cap)
        else:
            k, v, ks, vs = _alloc(S, cap, fmt)
            idx = torch.zeros((S, cap, 4, 128), dtype=torch.float32, device=DEV)
            cache = M.make_cache(k=k, v=v, idx_k=idx, kv_format=fmt, k_scale=ks, v_scale=vs)
        _append_all(cache, host, S, cap, dims)
        out = torch.empty((wl.n_q, 64, 128), device=DEV)
        ws = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_ATTEND_DECODE, wl.n_q, wl.max_pos), 256),
                         dtype=torch.uint8, device=DEV)
        M.msa_attend_decode(dims, cache, dev_bits(qs["q"], torch.bfloat16), dev(qs["stream"]), dev(qs["pos"]),
                            wl.max_pos, dev(o_sel), out, ws)
        # a prefill chunk of stream 1 (positions 1700 .. 1999) through the
        # quantized prefill path, whose rows also resolve through the table
        pre = pre_q[paged]
        ws_p = torch.empty(M.workspace_bytes(dims, M.MSA_OP_ATTEND_PREFILL, 300, 1999), dtype=torch.uint8,
                           device=DEV)
        M.msa_attend_prefill(dims, cache, pre["q"], 1, 1700, pre["sel"], pre["out"], ws_p)
        torch.cuda.synchronize()
        outs.append((out.cpu(), pre["out"].cpu()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
