"""paged_attn_decode_noalloc (the allocation-free variant of paged_attn_decode,
whose chunk records live in the library's fixed per-GPU scratch) against
paged_attn_decode with a caller workspace: two calls in a row, the second with
fewer rows, each giving the same bits and leaving the same pool bytes; a call
needing more scratch than the library holds is refused before anything
runs."""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import gpu_harness
    return gpu_harness


def _call(H, pkd, pool, seq, pos, q, k, v, distinct, noalloc):
    w = pool.w
    s, p = H.rows_tensors(seq, pos)
    n = s.numel()
    rows = pkd.make_rows(s, p, distinct)
    out = torch.full((n, w.n_q, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        pkd.paged_attn_decode_noalloc(pool.handle, rows, w.n_q, q, k, v, out, wl.F32)
    else:
        ws = H.aligned_empty(pkd.pkd_attn_workspace_bytes(pool.handle, w.n_q, n))
        pkd.paged_attn_decode(pool.handle, rows, w.n_q, q, k, v, out, wl.F32, ws)
    torch.cuda.synchronize()
    pkd.pkd_pool_check(pool.handle)
    return out.cpu()


@pytest.mark.parametrize("kvt,chunk,distinct", [(wl.BF16, 2, True), (wl.BF16, 3, False), (wl.FP8, 2, True)])
def test_noalloc_matches_workspace_entry_point(H, kvt, chunk, distinct):
    import paged_kv_decode_attn_amd as pkd
    assert pkd.pkd_attn_noalloc_scratch_bytes() == 64 << 20
    lens = (1, 40, 300, 129, 77, 520)
    w = wl.make("attn", "cpu", seed=41 + kvt + chunk, n_q=14, n_kv=2, d=128, kv_dtype=kvt, lens=lens, append=True,
                chunk=chunk, extra_pages=1)
    q, k, v = w.q.cuda(), w.k_new.cuda(), w.v_new.cuda()
    pools = {flag: H.GpuPool(w) for flag in (False, True)}
    # first call: every row; second call: three rows (fewer chunk records than the first left behind)
    sub = np.asarray([5, 0, 2])
    for rows in (np.arange(len(lens)), sub):
        outs = {}
        for flag in (False, True):
            outs[flag] = _call(H, pkd, pools[flag], w.seq[rows], w.pos[rows],
                               q[torch.as_tensor(rows)].contiguous(), k[torch.as_tensor(rows)].contiguous(),
                               v[torch.as_tensor(rows)].contiguous(), distinct, flag)
        assert torch.isfinite(outs[True]).all()
        assert torch.equal(outs[True].view(torch.int32), outs[False].view(torch.int32))
        assert torch.equal(pools[True].pages_bytes(), pools[False].pages_bytes())


def test_noalloc_refuses_beyond_scratch(H):
    import paged_kv_decode_attn_amd as pkd
    # 16 query heads of d 128 over 4,096 one-page chunks: 34 MB of chunk records per row
    desc = pkd.pkd_pool_desc(4, 32, 1, 128, wl.BF16, 1.0, 1.0, 2, 4096, 1)
    mem = H.aligned_empty(pkd.pkd_pool_bytes(desc))
    h = pkd.kv_pool_create(desc, mem)
    try:
        n = 2
        need = pkd.pkd_attn_workspace_bytes(h, 16, n)
        assert need > pkd.pkd_attn_noalloc_scratch_bytes() >= pkd.pkd_attn_workspace_bytes(h, 16, 1)
        s = torch.zeros(n, dtype=torch.int32, device="cuda")
        q = torch.zeros((n, 16, 128), dtype=torch.int16, device="cuda")
        out = torch.full((n, 16, 128), 7, dtype=torch.int16, device="cuda")
        with pytest.raises(pkd.PkdError) as ei:
            pkd.paged_attn_decode_noalloc(h, pkd.make_rows(s, s), 16, q, None, None, out, wl.BF16)
        assert ei.value.status == 3 and ei.value.needed == need
        assert ei.value.available == pkd.pkd_attn_noalloc_scratch_bytes()
        torch.cuda.synchronize()
        assert bool((out == 7).all())  # nothing ran
    finally:
        pkd.kv_pool_destroy(h)
