"""Host-side tests of the C ABI (no GPU needed, nothing is launched).

* libmsa_hip.so loads and exports every function include/msa.h declares;
* every entry point validates its host-visible arguments and returns the
  documented msa_status before touching the GPU (fake, never dereferenced
  pointers are used, so a validation bug that let a call through would be
  an error launch on this GPU-less host and show up as MSA_ERR_HIP);
* empty calls (n_q = 0) return MSA_OK without launching;
* workspace sizes follow the documented layouts.
"""
import ctypes
import os
import re

import pytest

import block_sparse_attention_msa_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, RANGE, ALIGN, WS, UNSUP = 0, -1, -2, -3, -4, -5, -6
A = ctypes.c_void_p(0x10000)     # fake 16-byte-aligned device address (never dereferenced)
B = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)   # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.LIB_PATH):
        from block_sparse_attention_msa_amd import build
        build.build()
    return M.lib()


def _cache(cap=4096, n_stream=2, idx=A, dsa=A):
    return M.Cache(idx, dsa, A, A, cap, n_stream)


def test_exports_every_declared_symbol(L):
    hdr = open(os.path.join(ROOT, "include", "msa.h")).read()
    declared = set(re.findall(r"^MSA_API [^(]*?\b(\w+)\(", hdr, flags=re.M))
    assert declared == set(M.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in (OK, NULL, SHAPE, RANGE, ALIGN, WS, UNSUP, -7):
        assert M.status_string(code).startswith("MSA_")


def test_dims_validation(L):
    c = _cache()
    for bad in (M.Dims(8, 16, 128, 128, 128, 16, 0.08), M.Dims(4, 8, 128, 128, 128, 16, 0.08),
                M.Dims(4, 16, 64, 128, 128, 16, 0.08), M.Dims(4, 16, 128, 64, 128, 16, 0.08),
                M.Dims(4, 16, 128, 128, 64, 16, 0.08), M.Dims(4, 16, 128, 128, 128, 0, 0.08),
                M.Dims(4, 16, 128, 128, 128, 65, 0.08), M.Dims(4, 16, 128, 128, 128, 16, 0.0),
                M.Dims(4, 16, 128, 128, 128, 16, float("nan"))):
        rc = L.msa_select(ctypes.byref(bad), ctypes.byref(c), A, A, A, 1, 100, A, A, A, 1 << 30, None)
        assert rc == UNSUP
    # DSA needs block 1 and 1 <= top_k <= 4096
    d = M.msa_dims()
    assert L.dsa_select(ctypes.byref(d), ctypes.byref(c), A, A, A, 1, 100, A, A, A, 1 << 30, None) == UNSUP
    assert L.msa_select(None, ctypes.byref(c), A, A, A, 1, 100, A, A, A, 1 << 30, None) == NULL


def test_null_misaligned_and_range(L):
    d = M.msa_dims()
    c = _cache()
    args = lambda **kw: [kw.get("idx_q", A), kw.get("stream", A), kw.get("pos", A), kw.get("n_q", 1),
                         kw.get("max_pos", 100), kw.get("sel", A), kw.get("n_sel", A), kw.get("ws", A),
                         kw.get("wsb", 1 << 30), None]
    sel = lambda **kw: L.msa_select(ctypes.byref(d), ctypes.byref(kw.pop("cache", c)), *args(**kw))
    assert sel(idx_q=None) == NULL
    assert sel(sel=None) == NULL
    assert sel(cache=_cache(idx=None)) == NULL
    assert sel(idx_q=MIS) == ALIGN
    assert sel(n_sel=MIS) == ALIGN
    assert sel(max_pos=4096) == RANGE          # == cap
    assert sel(max_pos=-1) == RANGE
    assert sel(n_q=-1) == SHAPE
    assert sel(cache=_cache(cap=0)) == SHAPE
    assert sel(cache=_cache(n_stream=0)) == SHAPE
    assert sel(ws=None) == NULL
    need = M.workspace_bytes(d, M.MSA_OP_SELECT, 1, 100)
    assert sel(wsb=need - 1) == WS
    assert sel(wsb=need) != WS                 # exactly enough (fails later only for want of a GPU)
    assert sel(n_q=0) == OK                    # empty call, nothing launched
    assert sel(n_q=0, ws=None) == OK


def test_prefill_range_checks(L):
    d = M.msa_dims()
    c = _cache(cap=1000, n_stream=2)
    f = lambda stream, pos0, n: L.msa_select_prefill(ctypes.byref(d), ctypes.byref(c), A, stream, pos0, n,
                                                     A, A, A, 1 << 30, None)
    assert f(2, 0, 10) == RANGE
    assert f(-1, 0, 10) == RANGE
    assert f(0, -1, 10) == RANGE
    assert f(0, 991, 10) == RANGE              # last position 1000 == cap
    assert f(0, 990, 0) == OK
    assert f(0, 0, -5) == SHAPE
    need = M.workspace_bytes(d, M.MSA_OP_SELECT_PREFILL, 10, 999)
    fw = lambda wsb: L.msa_select_prefill(ctypes.byref(d), ctypes.byref(c), A, 0, 990, 10, A, A, A, wsb, None)
    assert fw(need - 1) == WS
    assert fw(need) != WS
    need = M.workspace_bytes(d, M.MSA_OP_BLOCK_SCORES_PREFILL, 10, 999)
    fb = lambda wsb: L.msa_block_scores_prefill(ctypes.byref(d), ctypes.byref(c), A, 0, 990, 10, A, 8, A, wsb, None)
    assert fb(need - 1) == WS
    assert fb(need) != WS
    g = lambda n: L.msa_attend_prefill(ctypes.byref(d), ctypes.byref(c), A, 0, 990, n, A, A, A, 1 << 30,
                                       None)
    assert g(11) == RANGE
    assert g(0) == OK
    # more than 4096 blocks of 128 keys are beyond prefill attention's block masks
    big = _cache(cap=4097 * 128, n_stream=1)
    h = lambda pos0, n: L.msa_attend_prefill(ctypes.byref(d), ctypes.byref(big), A, 0, pos0, n, A, A, A, 0, None)
    assert h(4096 * 128 - 8, 8) != UNSUP      # last block 4095: accepted (fails later only for want of a GPU)
    assert h(4096 * 128 - 8, 9) == UNSUP
    # the step lists need workspace
    c1 = _cache(cap=1000, n_stream=1)
    need = M.workspace_bytes(d, M.MSA_OP_ATTEND_PREFILL, 10, 99)
    w = lambda ws, n: L.msa_attend_prefill(ctypes.byref(d), ctypes.byref(c1), A, 0, 90, 10, A, A, ws, n, None)
    assert w(None, need) == NULL
    assert w(A, need - 1) == WS


def test_append_validation(L):
    d = M.msa_dims()
    c = _cache(idx=None)
    f = lambda *src, n=1, max_pos=5: L.msa_index_append(ctypes.byref(d), ctypes.byref(c), A, A, n,
                                                       max_pos, *src, None)
    assert f(A, None, None) == NULL            # idx source but no idx cache
    assert f(None, MIS, None) == ALIGN
    assert f(None, A, A, n=0) == OK
    assert f(None, A, A, max_pos=4096) == RANGE
    dd = M.dsa_dims()
    cd = _cache(dsa=None)
    assert L.dsa_index_append(ctypes.byref(dd), ctypes.byref(cd), A, A, 1, 5, A, None, None, None) == NULL


def test_fp16_index_cache_validation(L):
    d = M.msa_dims()
    both = M.Cache(A, A, A, A, 4096, 2, B)           # f32 and fp16 index caches at once
    f16 = M.Cache(None, A, A, A, 4096, 2, B)         # fp16 only
    f16_mis = M.Cache(None, A, A, A, 4096, 2, MIS)
    sel = lambda c: L.msa_select(ctypes.byref(d), ctypes.byref(c), A, A, A, 1, 100, A, A, A, 1 << 30, None)
    assert sel(both) == UNSUP
    assert sel(f16) != UNSUP and sel(f16) not in (NULL, ALIGN)   # accepted (fails later only for want of a GPU)
    assert sel(f16_mis) == ALIGN
    assert L.msa_block_scores(ctypes.byref(d), ctypes.byref(both), A, A, A, 1, 100, A, 1, None) == UNSUP
    assert L.msa_select_prefill(ctypes.byref(d), ctypes.byref(both), A, 0, 0, 10, A, A, A, 1 << 30, None) == UNSUP
    assert L.msa_block_scores_prefill(ctypes.byref(d), ctypes.byref(both), A, 0, 0, 10, A, 1, A, 1 << 30,
                                      None) == UNSUP
    app = lambda c: L.msa_index_append(ctypes.byref(d), ctypes.byref(c), A, A, 1, 5, A, None, None, None)
    assert app(both) == UNSUP
    assert app(f16_mis) == ALIGN


def test_block_table_validation(L):
    d = M.msa_dims()
    ok = M.Cache(A, None, A, A, 4096, 2, None, B, 32)        # 32 pages of 128 cover cap 4096
    odd = ctypes.c_void_p(0x20002)                           # table entries are int32: 4-byte alignment
    mis = M.Cache(A, None, A, A, 4096, 2, None, odd, 32)
    short = M.Cache(A, None, A, A, 4097, 2, None, B, 32)     # cap beyond stride * 128
    zero = M.Cache(A, None, A, A, 4096, 2, None, B, 0)
    sel = lambda c: L.msa_select(ctypes.byref(d), ctypes.byref(c), A, A, A, 1, 100, A, A, A, 1 << 30, None)
    assert sel(ok) not in (NULL, ALIGN, SHAPE, UNSUP)       # accepted (fails later only for want of a GPU)
    assert sel(mis) == ALIGN
    assert sel(short) == SHAPE
    assert sel(zero) == SHAPE
    app = lambda c: L.msa_index_append(ctypes.byref(d), ctypes.byref(c), A, A, 1, 5, A, None, None, None)
    assert app(mis) == ALIGN and app(short) == SHAPE
    att = lambda c: L.msa_attend_prefill(ctypes.byref(d), ctypes.byref(c), A, 0, 0, 10, A, A, A, 1 << 30, None)
    assert att(mis) == ALIGN and att(zero) == SHAPE
    dd = M.dsa_dims()
    dsa_mis = M.Cache(None, A, A, A, 4096, 2, None, odd, 32)
    assert L.dsa_select(ctypes.byref(dd), ctypes.byref(dsa_mis), A, A, A, 1, 100, A, A, A, 1 << 30, None) == ALIGN


def test_dsa_select_heads_validation(L):
    dd = M.dsa_dims()
    c = M.Cache(None, A, A, A, 4096, 2, None, None, 0)
    call = lambda nh, w=A, q=A: L.dsa_select_heads(ctypes.byref(dd), ctypes.byref(c), q, w, nh, A, A, 1, 100,
                                                   A, A, A, 1 << 30, None)
    for nh in (0, 8, 20, 80, -16):
        assert call(nh) == UNSUP
    assert call(32, w=None) == NULL
    assert call(32, w=MIS) == ALIGN
    assert call(32) not in (NULL, ALIGN, SHAPE, UNSUP)     # accepted (fails later only for want of a GPU)
    md = M.msa_dims()
    assert L.dsa_select_heads(ctypes.byref(md), ctypes.byref(c), A, A, 32, A, A, 1, 100, A, A, A, 1 << 30,
                              None) == UNSUP                # MSA geometry


def test_index_project_validation(L):
    d = M.msa_dims()
    c = M.Cache(A, None, A, A, 4096, 2, None, None, 0)
    call = lambda pr, n=4, ws=1 << 30: L.msa_index_project(ctypes.byref(d), ctypes.byref(c), ctypes.byref(pr), A, A,
                                                             A, n, 100, A, A, ws, None)
    ok = M.Proj(768, A, A, A, A, 1e-6, 10000.0, 64)
    assert call(ok) not in (NULL, ALIGN, SHAPE, UNSUP, WS)        # accepted (fails later only for want of a GPU)
    for bad in (M.Proj(100, A, A, A, A, 1e-6, 1e4, 64), M.Proj(0, A, A, A, A, 1e-6, 1e4, 64),
                M.Proj(768, A, A, A, A, 1e-6, 1e4, 63), M.Proj(768, A, A, A, A, 1e-6, 1e4, 66),
                M.Proj(768, A, A, A, A, -1.0, 1e4, 64), M.Proj(768, A, A, A, A, 1e-6, 0.0, 64)):
        assert call(bad) == UNSUP
    assert call(M.Proj(768, None, A, A, A, 1e-6, 1e4, 64)) == NULL
    assert call(M.Proj(768, A, A, MIS, A, 1e-6, 1e4, 64)) == ALIGN
    assert call(ok, ws=16) == WS
    assert call(ok, n=0) == OK
    assert L.msa_index_project(ctypes.byref(d), ctypes.byref(c), None, A, A, A, 4, 100, A, A, 1 << 30, None) == NULL
    # workspace: splits of the hidden size x tokens x 1024 f32
    assert M.workspace_bytes(d, M.MSA_OP_INDEX_PROJECT, 32, 0) == 32 * 32 * 1024 * 4
    assert M.workspace_bytes(d, M.MSA_OP_INDEX_PROJECT, 4096, 0) == 1 * 4096 * 1024 * 4
    assert M.workspace_bytes(d, M.MSA_OP_INDEX_PROJECT, 1000, 0) == 2 * 1000 * 1024 * 4


def test_kv_format_validation(L):
    d = M.msa_dims()
    mk = lambda fmt, ks, vs: M.Cache(A, None, A, A, 4096, 2, None, None, 0, fmt, ks, vs)
    att = lambda c: L.msa_attend_decode(ctypes.byref(d), ctypes.byref(c), A, A, A, 1, 100, A, A, A, 1 << 30, None)
    assert att(mk(3, A, A)) == UNSUP and att(mk(-1, A, A)) == UNSUP
    assert att(mk(1, None, A)) == NULL
    assert att(mk(2, A, MIS)) == ALIGN
    assert att(mk(1, A, A)) not in (NULL, ALIGN, SHAPE, UNSUP)     # accepted (fails later only for want of a GPU)
    pre = lambda c: L.msa_attend_prefill(ctypes.byref(d), ctypes.byref(c), A, 0, 0, 10, A, A, A, 1 << 30, None)
    assert pre(mk(1, A, A)) not in (NULL, ALIGN, SHAPE, UNSUP)     # accepted (fails later only for want of a GPU)
    assert pre(mk(0, None, None)) not in (NULL, ALIGN, SHAPE, UNSUP)
    assert pre(mk(2, None, A)) == NULL and pre(mk(3, A, A)) == UNSUP
    # the quantized path checks the same workspace amount
    need = M.workspace_bytes(d, M.MSA_OP_ATTEND_PREFILL, 10, 9)
    pw = lambda c, n: L.msa_attend_prefill(ctypes.byref(d), ctypes.byref(c), A, 0, 0, 10, A, A, A, n, None)
    assert pw(mk(1, A, A), need - 1) == WS and pw(mk(2, A, A), need - 1) == WS
    assert pw(mk(1, A, A), need) != WS


def test_topk_block_limit(L):
    d = M.msa_dims()
    # 4096 blocks of 128 is the most a top-k wave ranks
    assert L.msa_topk_blocks(ctypes.byref(d), A, 4097, A, 1, 4096 * 128, A, A, None) == UNSUP
    assert L.msa_topk_blocks(ctypes.byref(d), A, 10, A, 1, 4096, A, A, None) == SHAPE   # stride < nblk
    assert L.msa_topk_blocks(ctypes.byref(d), A, 33, A, 0, 4095, A, A, None) == OK


def test_workspace_sizes(L):
    d = M.msa_dims()
    # select: n_q * 4 groups * nblk floats, 256-byte aligned
    assert M.workspace_bytes(d, M.MSA_OP_SELECT, 32, 32767) == 32 * 4 * 256 * 4
    assert M.workspace_bytes(d, M.MSA_OP_SELECT, 1, 0) == 256
    # prefill select: the block scores, then the keys split into bf16 high
    # and low parts (4 groups x 512 B per key)
    assert M.workspace_bytes(d, M.MSA_OP_SELECT_PREFILL, 4096, 32767) == 4096 * 4 * 256 * 4 + 32768 * 4 * 512
    assert M.workspace_bytes(d, M.MSA_OP_BLOCK_SCORES_PREFILL, 4096, 32767) == 32768 * 4 * 512
    assert M.workspace_bytes(d, M.MSA_OP_BLOCK_SCORES_PREFILL, 1, 100) == 101 * 4 * 512
    # attention partials: per (query, group, split) 16 heads x (128 + 2) floats
    n = M.workspace_bytes(d, M.MSA_OP_ATTEND_DECODE, 32, 32767)
    assert n % (16 * 130 * 4 * 4 * 32) == 0 and n > 0
    # prefill attention (every cache format): per (32-query tile, group) a
    # step count (256-byte aligned array), a used flag per (group, block)
    # (256-byte aligned), up to 32 * top_k 16-byte step entries (256-byte
    # aligned) and K and V of every block rearranged as bf16 (64 KiB per
    # group and block)
    def up(x):
        return -(-x // 256) * 256

    def prefill(n, max_pos=32767):
        nblk = max_pos // 128 + 1
        n_wg = -(-n // 32) * 4
        return up(up(n_wg * 4) + up(4 * nblk * 4) + up(n_wg * 32 * 16 * 16) + 4 * nblk * 2 * 128 * 128 * 2)

    assert prefill(4096) == 2048 + 4096 + 512 * 32 * 16 * 16 + 4 * 256 * 65536   # K and V of 256 blocks
    assert prefill(1, 127) == 256 + 256 + 4 * 8192 + 4 * 65536        # one query over one block
    for n in (1, 33, 100, 256, 257, 300, 4096, 4100):
        assert M.workspace_bytes(d, M.MSA_OP_ATTEND_PREFILL, n, 32767) == prefill(n), n
        assert M.workspace_bytes(d, M.MSA_OP_ATTEND_PREFILL, n, n - 1) == prefill(n, n - 1), n
    dd = M.dsa_dims()
    # DSA select: the f32 score rows (max_pos + 1 rounded up to 64); calls of
    # at most 32 queries over 8193 .. 65536 keys add, 256-byte aligned, the
    # chunk histograms (4096 u16 per 8192-key chunk), four ints, 4096 above-bin
    # ids and a boundary list of (key, id) per query
    assert M.workspace_bytes(dd, M.DSA_OP_SELECT, 33, 65535) == 33 * 65536 * 4
    assert M.workspace_bytes(dd, M.DSA_OP_SELECT, 16, 70000) == 16 * 70016 * 4
    assert M.workspace_bytes(dd, M.DSA_OP_SELECT, 16, 8191) == 16 * 8192 * 4
    assert M.workspace_bytes(dd, M.DSA_OP_SELECT, 16, 65535) == (
        16 * 65536 * 4 + 16 * 8 * 4096 * 2 + 256 + 16 * 4096 * 4 + 16 * 65536 * 4 + 16 * 65536 * 4)
    assert M.workspace_bytes(dd, M.DSA_OP_SELECT, 1, 8192) == (
        up(8256 * 4) + up(2 * 4096 * 2) + 256 + up(4096 * 4) + up(8256 * 4) + 8256 * 4)
    with pytest.raises(M.MsaError):
        M.workspace_bytes(d, M.DSA_OP_SELECT, 16, 65535)   # DSA op needs DSA dims


def test_workspace_of_an_empty_call_is_zero(L):
    """n_q == 0 is a valid empty call for every op: its workspace query
    returns 0 bytes (it used to divide by the number of (query, group)
    pairs on the host)."""
    d, dd = M.msa_dims(), M.dsa_dims()
    msa_ops = (M.MSA_OP_SELECT, M.MSA_OP_SELECT_PREFILL, M.MSA_OP_ATTEND_DECODE, M.MSA_OP_ATTEND_PREFILL,
               M.MSA_OP_BLOCK_SCORES_PREFILL, M.MSA_OP_INDEX_PROJECT, M.MSA_OP_DECODE_STEP)
    for op in msa_ops:
        for max_pos in (0, 127, 32767):
            assert M.workspace_bytes(d, op, 0, max_pos) == 0, (op, max_pos)
    for op in (M.DSA_OP_SELECT, M.DSA_OP_ATTEND_DECODE):
        assert M.workspace_bytes(dd, op, 0, 65535) == 0, op


def test_attend_decode_takes_token_ids(L):
    """msa_attend_decode with dims.block == 1 is the token-id (DSA) form:
    its dims are validated as DSA dims and its workspace is the DSA one."""
    c = _cache()
    dd = M.dsa_dims(2048)
    n_ws = M.workspace_bytes(dd, M.DSA_OP_ATTEND_DECODE, 16, 65535)
    assert M.workspace_bytes(dd, M.MSA_OP_ATTEND_DECODE, 16, 65535) == n_ws
    big = _cache(cap=65536, n_stream=16)
    args = lambda ws, wsb, d: [ctypes.byref(d), ctypes.byref(big), A, A, A, 16, 65535, A, B, ws, wsb, None]
    # past the dims check: a short workspace is reported, as by dsa_attend_decode
    if n_ws:
        assert L.msa_attend_decode(*args(A, n_ws - 1, dd)) == WS
        assert L.dsa_attend_decode(*args(A, n_ws - 1, dd)) == WS
    bad = M.Dims(4, 16, 128, 128, 1, 4097, 0.08)
    assert L.msa_attend_decode(*args(A, 1 << 40, bad)) == UNSUP
    # block 128 still needs an MSA top_k
    assert L.msa_attend_decode(*args(A, 1 << 40, M.Dims(4, 16, 128, 128, 128, 2048, 0.08))) == UNSUP


def test_select_static_limits(L):
    """msa_select_static validates like msa_select and rejects, before any
    launch, a call whose block scores do not fit the library's array."""
    d = M.msa_dims()
    c = _cache(cap=1 << 20, n_stream=4)
    call = lambda n_q, max_pos, **kw: L.msa_select_static(ctypes.byref(d), ctypes.byref(c), kw.get("idx_q", A),
                                                          A, A, n_q, max_pos, A, B, None)
    limit = M.MSA_STATIC_SCRATCH_BYTES
    assert limit == 4 << 20
    # 1025 queries at 32K context: 1025 * 4 * 256 * 4 B > 4 MiB
    assert call(1025, 32767) == WS
    assert call(257, 131071) == WS
    assert call(1, 4095, idx_q=None) == NULL
    assert call(1, 4095, idx_q=MIS) == ALIGN
    assert call(0, 4095) == OK
    assert call(1, 1 << 20) == RANGE


def test_decode_step_validation_and_workspace(L):
    """msa_decode_step: the block scores of msa_select followed by the
    attention partials of msa_attend_decode (each 256-byte aligned); the
    index keys to append are required, K/V rows optional; the usual checks
    run before any launch."""
    d = M.msa_dims()
    up = lambda x: -(-x // 256) * 256
    for n_q, max_pos in ((1, 4095), (5, 2999), (32, 32767), (20, 8191), (100, 127)):
        sel_ws = M.workspace_bytes(d, M.MSA_OP_SELECT, n_q, max_pos)
        att_ws = M.workspace_bytes(d, M.MSA_OP_ATTEND_DECODE, n_q, max_pos)
        assert M.workspace_bytes(d, M.MSA_OP_DECODE_STEP, n_q, max_pos) == sel_ws + up(att_ws) + up(n_q * 4 * 4)
    c = _cache(dsa=None)
    need = M.workspace_bytes(d, M.MSA_OP_DECODE_STEP, 1, 4095)

    def step(idx_new=A, k_new=A, v_new=A, n=1, max_pos=4095, ws=A, nb=need, cache=c):
        return L.msa_decode_step(ctypes.byref(d), ctypes.byref(cache), A, A, n, max_pos, idx_new, k_new, v_new,
                                 A, A, A, A, A, ws, nb, None)
    assert step(n=0) == OK
    assert step(idx_new=None) == NULL
    assert step(k_new=MIS) == ALIGN
    assert step(ws=None) == NULL
    assert step(nb=need - 1) == WS
    assert step(max_pos=4096) == RANGE
    assert step(n=-1) == SHAPE
    assert step(cache=_cache(idx=None, dsa=None)) == NULL        # no index cache
    assert step(k_new=None, v_new=None) not in (NULL, ALIGN, SHAPE, UNSUP, WS)   # accepted (no GPU here)


def test_call_size_limits(L):
    """Calls larger than the launch grids allow are refused before any
    launch: more than MSA_MAX_QUERIES queries per select / block-score /
    top-k / attention / step call (65535 for the DSA selections), more than
    MSA_MAX_ROWS rows per append or projection call; the workspace query
    refuses them too.  The limits are
    the header's (parsed from include/msa.h)."""
    hdr = open(os.path.join(ROOT, "include", "msa.h")).read()
    mq = int(re.search(r"#define MSA_MAX_QUERIES \(\(int64_t\)1 << (\d+)\)", hdr).group(1))
    mr = int(re.search(r"#define MSA_MAX_ROWS \(\(int64_t\)1 << (\d+)\)", hdr).group(1))
    assert (1 << mq, 1 << mr) == (M.MSA_MAX_QUERIES, M.MSA_MAX_ROWS)
    Q, R = M.MSA_MAX_QUERIES, M.MSA_MAX_ROWS
    # the attention launch's widest grid (4 groups x 8 splits of 256 threads
    # per query) and the append's (128 threads per row) fit one dimension
    assert Q * 4 * 8 * 256 < 1 << 32 and R * 128 < 1 << 32
    d, dd = M.msa_dims(), M.dsa_dims(2048)
    c = _cache(cap=1 << 20, n_stream=1)
    big = 1 << 30
    calls = {
        "msa_select": lambda n: L.msa_select(ctypes.byref(d), ctypes.byref(c), A, A, A, n, 100, A, A, A, big, None),
        "msa_block_scores": lambda n: L.msa_block_scores(ctypes.byref(d), ctypes.byref(c), A, A, A, n, 100, A, 8,
                                                         None),
        "msa_topk_blocks": lambda n: L.msa_topk_blocks(ctypes.byref(d), A, 8, A, n, 100, A, A, None),
        "msa_attend_decode": lambda n: L.msa_attend_decode(ctypes.byref(d), ctypes.byref(c), A, A, A, n, 100, A, A,
                                                           A, big, None),
        "dsa_select": lambda n: L.dsa_select(ctypes.byref(dd), ctypes.byref(c), A, A, A, n, 100, A, A, A, big,
                                             None),
        "dsa_select_heads": lambda n: L.dsa_select_heads(ctypes.byref(dd), ctypes.byref(c), A, A, 32, A, A, n, 100,
                                                         A, A, A, big, None),
        "msa_select_prefill": lambda n: L.msa_select_prefill(ctypes.byref(d), ctypes.byref(c), A, 0, 0, n, A, A, A,
                                                             big, None),
        "msa_attend_prefill": lambda n: L.msa_attend_prefill(ctypes.byref(d), ctypes.byref(c), A, 0, 0, n, A, A, A,
                                                             big, None),
        "msa_decode_step": lambda n: L.msa_decode_step(ctypes.byref(d), ctypes.byref(c), A, A, n, 100, A, A, A, A,
                                                       A, A, A, A, A, big, None),
    }
    for name, f in calls.items():
        lim = 65535 if name.startswith("dsa_") else Q     # the DSA scans' query grid dimension
        assert f(lim + 1) == UNSUP, name
        assert f(lim) != UNSUP, name         # at the limit: accepted (fails later only for want of a GPU)
    app = lambda n: L.msa_index_append(ctypes.byref(d), ctypes.byref(c), A, A, n, 100, A, A, A, None)
    assert app(R + 1) == UNSUP
    assert app(R) != UNSUP
    bad = ctypes.c_size_t(-1).value
    for op in (M.MSA_OP_SELECT, M.MSA_OP_ATTEND_DECODE, M.MSA_OP_ATTEND_PREFILL, M.MSA_OP_DECODE_STEP):
        assert L.msa_workspace_bytes(ctypes.byref(d), op, Q + 1, 100) == bad, op
        assert L.msa_workspace_bytes(ctypes.byref(d), op, Q, 100) < 1 << 40, op
    assert L.msa_workspace_bytes(ctypes.byref(d), M.MSA_OP_INDEX_PROJECT, R + 1, 100) == bad
    assert L.msa_workspace_bytes(ctypes.byref(d), M.MSA_OP_INDEX_PROJECT, R, 100) < 1 << 40
