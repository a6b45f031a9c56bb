"""msa_select_static (no workspace, block scores in the library's per-device
array) against msa_select on the same inputs, through the C ABI: two calls in
a row, the second smaller than the first, then a call too large for the
array (rejected on the host, nothing launched)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_msa_amd as M
import workloads as W
from _gpu_common import DEV, GpuWorkload, dev, log

pytestmark = pytest.mark.gpu


def _both(gw: GpuWorkload, dims, idx):
    qs = gw.qs
    n_q = len(idx)
    st, ps = dev(qs["stream"][idx]), dev(qs["pos"][idx])
    max_pos = int(qs["pos"][idx].max())
    iq = dev(qs["idx_q"][idx])
    sel_a = torch.full((n_q, 4, dims.top_k), -5, dtype=torch.int32, device=DEV)
    nsel_a = torch.full((n_q, 4), -5, dtype=torch.int32, device=DEV)
    sel_b, nsel_b = sel_a.clone(), nsel_a.clone()
    ws = torch.empty(max(M.workspace_bytes(dims, M.MSA_OP_SELECT, n_q, max_pos), 256), dtype=torch.uint8,
                     device=DEV)
    M.msa_select(dims, gw.cache, iq, st, ps, max_pos, sel_a, nsel_a, ws)
    M.msa_select_static(dims, gw.cache, iq, st, ps, max_pos, sel_b, nsel_b)
    torch.cuda.synchronize()
    return sel_a.cpu().numpy(), nsel_a.cpu().numpy(), sel_b.cpu().numpy(), nsel_b.cpu().numpy()


def test_select_static_equals_select():
    # 24 queries over 6 streams at up to 24K context, then 5 queries at most
    # 3K into the same array (its earlier contents must not leak through)
    rng = np.random.default_rng(5)
    cap = 24576
    pos = np.concatenate([[cap - 1, 0, 127, 128, 3000], rng.integers(0, cap, 19)]).astype(np.int32)
    wl = W.Workload("static", "msa_decode", 6, cap, tuple(int(i % 6) for i in range(24)), tuple(int(p) for p in pos))
    gw = GpuWorkload(wl)
    dims = M.msa_dims(16, W.SCALE)
    few = np.array([i for i in range(24) if wl.pos[i] <= 3000][:5])     # includes positions 0, 127, 128, 3000
    for name, idx in (("24 queries, max_pos 24575", np.arange(24)), (f"{len(few)} queries, max_pos <= 3000", few)):
        log(f"[select_static] {name}")
        a, na, b, nb = _both(gw, dims, idx)
        assert np.array_equal(a, b), name
        assert np.array_equal(na, nb), name
        assert (na >= 1).all()


def test_select_static_rejects_oversized_call():
    wl = W.decode_workload("static_big", 2, 4096)
    gw = GpuWorkload(wl)
    dims = M.msa_dims(16, W.SCALE)
    n_q = M.MSA_STATIC_SCRATCH_BYTES // (4 * 32 * 4) + 1       # one query too many at 32 blocks
    z = torch.zeros(n_q, dtype=torch.int32, device=DEV)
    iq = torch.zeros((n_q, 4, 128), dtype=torch.float32, device=DEV)
    sel = torch.full((n_q, 4, 16), -5, dtype=torch.int32, device=DEV)
    nsel = torch.full((n_q, 4), -5, dtype=torch.int32, device=DEV)
    with pytest.raises(M.MsaError) as e:
        M.msa_select_static(dims, gw.cache, iq, z, z + 4095, 4095, sel, nsel)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert int((sel != -5).sum()) == 0 and int((nsel != -5).sum()) == 0
