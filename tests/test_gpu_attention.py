"""Parity of the HIP paged attention (with and without the append of the row's
own token) against the fp64 oracle, element by element; bit-identity across
batch compositions and runs; invalid rows; chunked and unchunked reduction."""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

# Tolerances: the kernel reads the same stored codes as the oracle and reduces
# in fp32 (scores by the matrix core, weights as a hi + lo bf16 pair with ~16
# significant bits), so the attention output agrees to ~1e-5 relative;
# 1e-4 leaves a margin of ~10x.  Outputs stored in bf16 add one rounding of
# at most 2^-8 relative.
TOL_F32_OUT = 1e-4
TOL_BF16_OUT = 2 ** -8 + 1e-4


@pytest.fixture(scope="module")
def H():
    import gpu_harness
    return gpu_harness


def oracle_attn(orc, w, seq, pos, q, k_new=None, v_new=None):
    hk, hv = wl.history_lists(w)
    hist = orc.History(hk, hv, w.kv_dtype, w.n_kv, w.head_dim)
    qd = w.q_dtype
    tonp = lambda t: None if t is None else wl.to_numpy_codes(t, qd)
    return orc.attention(w.n_q, w.n_kv, w.head_dim, w.kv_dtype, w.k_scale, w.v_scale, hist, seq, pos, qd,
                         tonp(q), tonp(k_new), tonp(v_new))


CASES = [
    # (kv dtype, n_q, n_kv, d, append, chunk)
    (wl.F32, 4, 2, 64, True, 2),
    (wl.F32, 4, 2, 64, False, 8),
    (wl.BF16, 4, 2, 128, True, 2),
    (wl.BF16, 4, 2, 128, False, 8),
    (wl.BF16, 14, 2, 128, True, 1),
    (wl.BF16, 2, 2, 128, True, 3),
    (wl.BF16, 32, 2, 64, True, 2),
    (wl.FP8, 14, 2, 128, True, 2),
    (wl.FP8, 4, 2, 64, False, 8),
    (wl.BF16, 7, 1, 128, True, 8),
]


@pytest.mark.parametrize("kvt,nq,nkv,d,append,chunk", CASES)
def test_attention_parity(H, orc, kvt, nq, nkv, d, append, chunk):
    lens = (1, 2, 31, 32, 33, 63, 64, 65, 97, 160, 200)
    w = wl.make("attn", "cpu", seed=11 + nq + d + kvt, n_q=nq, n_kv=nkv, d=d, kv_dtype=kvt, lens=lens,
                append=append, chunk=chunk)
    print(f"case {w.name} append={append} chunk={chunk}", flush=True)
    pool = H.GpuPool(w)
    dev = lambda t: None if t is None else t.to("cuda")
    out = H.run_attention(pool, w.seq, w.pos, dev(w.q), dev(w.k_new), dev(w.v_new), wl.F32)
    want = oracle_attn(orc, w, w.seq, w.pos, w.q, w.k_new, w.v_new)
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    e = H.rel_err(got, want)
    print(f"  max rel err {e:.3e}")
    assert e <= TOL_F32_OUT
    # L = 1 (first row): the output is the value of token 0 (bit-exact outside fp8)
    if kvt != wl.FP8:
        assert np.array_equal(got[0], want[0])
    # bf16 output = RNE of the f32 output
    if kvt != wl.F32:
        if append:  # re-run from a fresh pool: the append must not be applied twice differently
            pool = H.GpuPool(w)
        ob = H.run_attention(pool, w.seq, w.pos, dev(w.q), dev(w.k_new), dev(w.v_new), wl.BF16)
        gb = H.values(ob, wl.BF16)
        assert H.rel_err(gb, want) <= TOL_BF16_OUT
        assert np.array_equal(gb, torch.from_numpy(got).float().to(torch.bfloat16).double().numpy())


FUSED_CASES = [
    # (kv dtype, n_q, n_kv, d): the append inside the attention kernel
    (wl.F32, 4, 2, 64),
    (wl.BF16, 4, 2, 128),
    (wl.BF16, 14, 2, 128),
    (wl.BF16, 32, 2, 64),
    (wl.FP8, 14, 2, 128),
    (wl.FP8, 4, 2, 64),
]


@pytest.mark.parametrize("chunk", [8, 2])
@pytest.mark.parametrize("kvt,nq,nkv,d", FUSED_CASES)
def test_fused_append_bit_identical(H, kvt, nq, nkv, d, chunk):
    """With every sequence appearing once, the append runs inside the attention
    kernel (the row's token substituted in registers).  Outputs and the pool
    bytes it leaves are bit-identical to the separate append followed by
    attention, for a token in every one of the 32 page slots."""
    lens = tuple(range(1, 41)) + (63, 64, 65, 96, 97, 128, 129)
    w = wl.make("attn", "cpu", seed=40 + nq + d + kvt, n_q=nq, n_kv=nkv, d=d, kv_dtype=kvt, lens=lens,
                append=True, chunk=chunk)  # 8: one chunk per row; 2: the row's last chunk appends
    dev = lambda t: t.to("cuda")
    outs, pools = [], []
    for distinct in (False, True):
        pool = H.GpuPool(w)
        outs.append(H.run_attention(pool, w.seq, w.pos, dev(w.q), dev(w.k_new), dev(w.v_new), wl.F32,
                                    distinct=distinct).cpu())
        pools.append(pool.pages_bytes().cpu())
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(pools[0], pools[1])
    # and a shuffled batch through the fused path gives the same bits per row
    perm = np.random.default_rng(5).permutation(w.n_rows)
    pool = H.GpuPool(w)
    sh = H.run_attention(pool, w.seq[perm], w.pos[perm], dev(w.q[perm]), dev(w.k_new[perm]), dev(w.v_new[perm]),
                         wl.F32, distinct=True).cpu()
    assert torch.equal(sh, outs[0][torch.as_tensor(perm)])


@pytest.mark.parametrize("kvt,nq,nkv,d,append", [
    (wl.BF16, 14, 2, 128, True), (wl.BF16, 4, 2, 128, False), (wl.FP8, 14, 2, 128, True),
    (wl.F32, 4, 2, 64, True), (wl.BF16, 32, 2, 64, False)])
def test_shared_prefix_staging(H, orc, kvt, nq, nkv, d, append):
    """Rows whose first page is one physical page: in a batch, each workgroup
    of four rows stages that page in LDS once; alone, a row reads it from HBM.
    The bits agree, and both match the oracle."""
    lens = (40, 50, 70, 100, 33, 64, 65, 129, 97)
    w = wl.make("attn", "cpu", seed=21 + nq + d + kvt, n_q=nq, n_kv=nkv, d=d, kv_dtype=kvt, lens=lens,
                append=append, chunk=8, shared_first_page=True)
    assert all(int(w.tables[s][0]) == int(w.tables[0][0]) for s in range(len(lens)))
    dev = lambda t: None if t is None else t.to("cuda")
    full = H.run_attention(H.GpuPool(w), w.seq, w.pos, dev(w.q), dev(w.k_new), dev(w.v_new), wl.F32,
                           distinct=True).cpu()
    want = oracle_attn(orc, w, w.seq, w.pos, w.q, w.k_new, w.v_new)
    assert H.rel_err(full.numpy().astype(np.float64), want) <= TOL_F32_OUT
    for r in range(len(lens)):
        sl = slice(r, r + 1)
        one = H.run_attention(H.GpuPool(w), w.seq[sl], w.pos[sl], dev(w.q[sl]),
                              None if w.k_new is None else dev(w.k_new[sl]),
                              None if w.v_new is None else dev(w.v_new[sl]), wl.F32, distinct=True).cpu()
        assert torch.equal(one[0], full[r]), r


def test_attention_batch_invariance(H):
    """A row gives the same bits alone, in the full batch, in a shuffled batch,
    in a subset, and on a repeated run; chunked and direct pools each."""
    for chunk in (2, 8):
        lens = (5, 33, 64, 65, 150, 199, 200, 256)
        w = wl.make("attn", "cpu", seed=3, n_q=14, n_kv=2, d=128, kv_dtype=wl.BF16, lens=lens, append=False,
                    chunk=chunk)
        pool = H.GpuPool(w)
        q = w.q.to("cuda")
        full = H.run_attention(pool, w.seq, w.pos, q).cpu()
        again = H.run_attention(pool, w.seq, w.pos, q).cpu()
        assert torch.equal(full, again)
        perm = np.asarray([6, 2, 7, 0, 5, 1, 4, 3])
        sh = H.run_attention(pool, w.seq[perm], w.pos[perm], q[torch.as_tensor(perm, device="cuda")]).cpu()
        assert torch.equal(sh, full[torch.as_tensor(perm)])
        for r in (0, 4, 7):
            one = H.run_attention(pool, w.seq[r:r + 1], w.pos[r:r + 1], q[r:r + 1]).cpu()
            assert torch.equal(one[0], full[r])
        # the same row repeated many times in one batch
        reps = np.full(300, 6, np.int32)
        many = H.run_attention(pool, w.seq[reps], w.pos[reps], q[6:7].expand(300, -1, -1).contiguous()).cpu()
        assert torch.equal(many, full[6:7].expand(300, -1, -1))


def test_attention_rows_of_one_sequence(H, orc):
    """Several rows of one sequence in one call (a prefill slice): all appends
    land before any read, so row p sees the tokens of rows < p."""
    w = wl.make("attn", "cpu", seed=5, n_q=4, n_kv=2, d=128, kv_dtype=wl.BF16, lens=(40,), append=True,
                chunk=2, extra_pages=3)
    # rows at positions 39..70 of sequence 0, with fresh k/v for each
    gen = torch.Generator().manual_seed(9)
    n = 32
    seq = np.zeros(n, np.int32)
    pos = np.arange(39, 39 + n, dtype=np.int32)
    q = wl.encode(torch.randn((n, 4, 128), generator=gen), wl.BF16)
    kn = wl.encode(torch.randn((n, 2, 128), generator=gen), wl.BF16)
    vn = wl.encode(torch.randn((n, 2, 128), generator=gen), wl.BF16)
    pool = H.GpuPool(w)
    out = H.run_attention(pool, seq, pos, q.cuda(), kn.cuda(), vn.cuda())
    want = oracle_attn(orc, w, seq, pos, q, kn, vn)
    assert H.rel_err(out.cpu().numpy(), want) <= TOL_F32_OUT
    # the pool now holds the appended tokens: read them back through the oracle's gather
    pages = pool.pages_bytes().cpu().numpy()
    k, v = orc.gather_history(pages, 2, 128, wl.BF16, w.tables[0], 39 + n)
    assert np.array_equal(k[39:].view(np.uint16), wl.to_numpy_codes(kn, wl.BF16))
    assert np.array_equal(v[39:].view(np.uint16), wl.to_numpy_codes(vn, wl.BF16))


def test_fp8_append_codes(H, orc):
    """The appended fp8 codes are E4M3 RNE(value / scale) with saturation,
    exactly as the oracle encodes them (values beyond the calibrated range
    included)."""
    w = wl.make("attn", "cpu", seed=6, n_q=4, n_kv=2, d=128, kv_dtype=wl.FP8, lens=(10, 45), append=True,
                chunk=2)
    gen = torch.Generator().manual_seed(1)
    kn = wl.encode(torch.randn((2, 2, 128), generator=gen) * 3.0, wl.BF16)  # some past 448 * scale
    vn = wl.encode(torch.randn((2, 2, 128), generator=gen) * 3.0, wl.BF16)
    pool = H.GpuPool(w)
    H.run_attention(pool, w.seq, w.pos, w.q.cuda(), kn.cuda(), vn.cuda())
    pages = pool.pages_bytes().cpu().numpy()
    for s in range(2):
        L = int(w.pos[s]) + 1
        k, v = orc.gather_history(pages, 2, 128, wl.FP8, w.tables[s], L)
        kv = orc.bf16_value(wl.to_numpy_codes(kn[s], wl.BF16))
        vv = orc.bf16_value(wl.to_numpy_codes(vn[s], wl.BF16))
        want_k = orc.e4m3_round((kv.astype(np.float32) / np.float32(w.k_scale)).astype(np.float64))
        want_v = orc.e4m3_round((vv.astype(np.float32) / np.float32(w.v_scale)).astype(np.float64))
        assert np.array_equal(k[L - 1], want_k)
        assert np.array_equal(v[L - 1], want_v)
        assert (k[L - 1] == 0x7E).any() or (k[L - 1] == 0xFE).any()  # saturation exercised


def test_invalid_rows_zeroed_and_reported(H):
    import paged_kv_decode_attn_amd as pkd
    for chunk in (1, 8):  # chunked and direct reduction
        w = wl.make("attn", "cpu", seed=7, n_q=4, n_kv=2, d=128, kv_dtype=wl.BF16, lens=(20, 40), append=False,
                    chunk=chunk, extra_pages=0)
        pool = H.GpuPool(w)
        seq = np.asarray([0, 5, 1, 1, -1], np.int32)
        pos = np.asarray([19, 3, 64, 39, 0], np.int32)  # seq 5 absent, pos 64 past 2 pages, seq -1
        q = torch.cat([w.q] * 3)[:5].cuda()
        out = H.run_attention(pool, seq, pos, q).cpu()
        assert torch.equal(out[1], torch.zeros_like(out[1]))
        assert torch.equal(out[2], torch.zeros_like(out[2]))
        assert torch.equal(out[4], torch.zeros_like(out[4]))
        assert out[0].abs().sum() > 0 and out[3].abs().sum() > 0
        with pytest.raises(pkd.PkdError) as ei:
            pkd.pkd_pool_check(pool.handle)
        assert ei.value.status == 7 and ei.value.needed == 3  # bad sequence and bad position
        pkd.pkd_pool_check(pool.handle)  # cleared


def test_invalid_rows_fused_append_and_flag_refusal(H):
    """Rows with a bad sequence or position are zeroed and reported on the
    fused-append path too (and append nothing); unknown row flags are refused
    before anything runs."""
    import paged_kv_decode_attn_amd as pkd
    w = wl.make("attn", "cpu", seed=9, n_q=4, n_kv=2, d=128, kv_dtype=wl.BF16, lens=(20, 40), append=True,
                chunk=8, extra_pages=0)
    pool = H.GpuPool(w)
    before = pool.pages_bytes().clone()
    seq = np.asarray([0, 5, -1], np.int32)
    pos = np.asarray([19, 3, 0], np.int32)
    q = torch.cat([w.q] * 2)[:3].cuda()
    kn = torch.cat([w.k_new] * 2)[:3].cuda()
    vn = torch.cat([w.v_new] * 2)[:3].cuda()
    out = H.run_attention(pool, seq, pos, q, kn, vn, distinct=True).cpu()
    assert torch.equal(out[1], torch.zeros_like(out[1])) and torch.equal(out[2], torch.zeros_like(out[2]))
    assert out[0].abs().sum() > 0
    with pytest.raises(pkd.PkdError) as ei:
        pkd.pkd_pool_check(pool.handle)
    assert ei.value.status == 7
    # only sequence 0's page 0 (its token 19) changed
    after = pool.pages_bytes()
    changed = torch.nonzero(after != before).flatten()
    blk = pool.info.block_bytes
    page0 = int(w.tables[0][0])
    assert changed.numel() > 0
    assert bool(((changed // (2 * 2 * blk)) == page0).all())
    s_t, p_t = H.rows_tensors(seq, pos)
    rows = pkd.pkd_rows(s_t.data_ptr(), p_t.data_ptr(), 3, 2)
    o2 = torch.empty_like(out).cuda()
    with pytest.raises(pkd.PkdError) as ei:
        pkd.paged_attn_decode(pool.handle, rows, 4, q, kn, vn, o2, 0,
                              H.aligned_empty(pkd.pkd_attn_workspace_bytes(pool.handle, 4, 3)))
    assert ei.value.status == 1


TABLE_CASES = [
    # lens, chunk, distinct, (bad sequence, its logical page), bad entry (0 = one past the pool, 1 = -1),
    # first page shared by the sequences (the staging kernel)
    ((100, 40, 70), 100, True, (0, 1), 0, False),     # one wave per row, fused append; first window
    ((100, 40, 70), 100, True, (0, 3), 1, False),     # the row's own page
    ((2600, 40, 70), 100, True, (0, 70), 0, False),   # a later window of a long row (reloaded in the page loop)
    ((2600, 40, 70), 100, False, (0, 81), 1, False),  # own page of a long row; separate append kernel
    ((100, 40, 70), 2, True, (0, 1), 1, False),       # page chunks, fused append in the last chunk, ordered merge
    ((100, 40, 70), 2, False, (0, 3), 0, False),      # page chunks, separate append kernel, own page
    ((100, 40, 70), 100, True, (2, 1), 0, True),      # shared leading pages staged in LDS
]


@pytest.mark.parametrize("lens,chunk,distinct,bad,kind,shared", TABLE_CASES)
def test_table_entry_outside_pool(H, lens, chunk, distinct, bad, kind, shared):
    """A block-table entry outside the pool, written into the device copy of
    the table behind block_table_set: the kernels never dereference it (page 0
    is read in its place and nothing outside the pool is written: the guard
    bytes around the pool keep their fill), the row's outputs are zeros and
    bit 4 of the error word is set; every other row keeps the bits of a
    clean run, and the pool's pages change only where a clean run changes
    them, plus possibly the bad row's own page."""
    import paged_kv_decode_attn_amd as pkd
    w = wl.make("attn", "cpu", seed=31, n_q=8, n_kv=2, d=128, kv_dtype=wl.BF16, lens=lens, append=True,
                chunk=chunk, extra_pages=0, shared_first_page=shared)
    s_bad, lp = bad
    assert lp < int(w.counts[s_bad])
    args = (w.seq, w.pos, w.q.cuda(), w.k_new.cuda(), w.v_new.cuda(), wl.F32, distinct)
    clean_pool = H.GpuPool(w)
    clean = H.run_attention(clean_pool, *args).cpu()
    pkd.pkd_pool_check(clean_pool.handle)
    assert (pkd.pkd_pool_info_get(clean_pool.handle).shared_pages > 0) == shared
    page_bytes = 2 * w.n_kv * clean_pool.info.block_bytes
    pool = H.GpuPool(w, pad=2 * page_bytes)
    pool.table_entries()[s_bad, lp] = w.num_pages if kind == 0 else -1
    torch.cuda.synchronize()
    out = H.run_attention(pool, *args).cpu()
    with pytest.raises(pkd.PkdError) as ei:
        pkd.pkd_pool_check(pool.handle)
    assert ei.value.status == 7 and ei.value.needed & 4
    assert pool.guard_intact()
    r_bad = int(np.nonzero(w.seq == s_bad)[0][0])
    assert (out[r_bad] == 0).all()
    others = [r for r in range(w.n_rows) if r != r_bad]
    assert torch.equal(out[others].view(torch.int32), clean[others].view(torch.int32))
    own = int(w.tables[s_bad][int(w.pos[r_bad]) // 32])
    a = pool.pages_bytes().view(w.num_pages, -1).cpu()
    b = clean_pool.pages_bytes().view(w.num_pages, -1).cpu()
    keep = [pg for pg in range(w.num_pages) if pg != own]
    assert torch.equal(a[keep], b[keep])
    pkd.pkd_pool_check(pool.handle)  # cleared


def test_block_table_refusals(H):
    import paged_kv_decode_attn_amd as pkd
    w = wl.make("attn", "cpu", seed=8, n_q=4, n_kv=2, d=64, kv_dtype=wl.F32, lens=(20, 40), append=False,
                chunk=2)
    pool = H.GpuPool(w)
    mp = w.max_pages_per_seq
    with pytest.raises(pkd.PkdError) as ei:
        pkd.block_table_set(pool.handle, 0, np.zeros((1, mp), np.int32), [mp + 1])
    assert ei.value.status == 4 and ei.value.needed == mp + 1 and ei.value.available == mp
    bad = np.zeros((1, mp), np.int32)
    bad[0, 0] = w.num_pages
    with pytest.raises(pkd.PkdError) as ei:
        pkd.block_table_set(pool.handle, 0, bad, [1])
    assert ei.value.status == 4 and ei.value.needed == w.num_pages and ei.value.available == w.num_pages
    dup = np.zeros((1, mp), np.int32)
    with pytest.raises(pkd.PkdError) as ei:
        pkd.block_table_set(pool.handle, 0, dup, [2])
    assert ei.value.status == 5
    with pytest.raises(pkd.PkdError) as ei:
        pkd.block_table_set(pool.handle, 1, w.tables, w.counts)
    assert ei.value.status == 4 and ei.value.needed == 3 and ei.value.available == 2
    # refused calls changed nothing: attention still matches a fresh pool
    out = H.run_attention(pool, w.seq, w.pos, w.q.cuda()).cpu()
    fresh = H.run_attention(H.GpuPool(w), w.seq, w.pos, w.q.cuda()).cpu()
    assert torch.equal(out, fresh)


def test_shared_page_count(H):
    """block_table_set keeps the count of physical pages that two or more
    sequences list (pkd_pool_info.shared_pages) exact as tables are set,
    replaced and cleared; a refused call leaves it unchanged."""
    import paged_kv_decode_attn_amd as pkd
    desc = pkd.pkd_pool_desc(8, 32, 1, 64, wl.BF16, 1.0, 1.0, 3, 4, 4)
    mem = H.aligned_empty(pkd.pkd_pool_bytes(desc))
    h = pkd.kv_pool_create(desc, mem)
    try:
        def shared():
            return pkd.pkd_pool_info_get(h).shared_pages

        def put(seq, pages):
            row = np.full((1, 4), -1, np.int32)
            row[0, :len(pages)] = pages
            pkd.block_table_set(h, seq, row, [len(pages)])

        assert shared() == 0
        put(0, [0, 1, 2])
        put(1, [0, 1, 3])
        assert shared() == 2          # pages 0 and 1
        put(2, [0, 4])
        assert shared() == 2          # page 0 now listed three times
        put(1, [5, 6])
        assert shared() == 1          # page 1 back to one sequence; page 0 still shared
        with pytest.raises(pkd.PkdError):
            put(1, [5, 5])            # duplicate in one table: refused, nothing changes
        assert shared() == 1
        put(2, [])
        assert shared() == 0
        both = np.array([[7, 0, -1, -1], [7, 1, -1, -1]], np.int32)
        pkd.block_table_set(h, 1, both, [2, 2])
        assert shared() == 3          # page 7 (sequences 1, 2), 0 (0, 1) and 1 (0, 2)
    finally:
        pkd.kv_pool_destroy(h)


@pytest.mark.parametrize("kvt,nq,nkv,d,append", [
    (wl.BF16, 28, 4, 128, True), (wl.FP8, 14, 2, 128, True), (wl.F32, 4, 2, 64, False)])
def test_staging_variant_bit_identical(H, kvt, nq, nkv, d, append):
    """The same logical pool with its first pages shared physically (the
    staging kernel runs) and with private copies of them (the kernel without
    LDS, whose workgroups take four (row, kv head) units) gives the same bits."""
    import dataclasses
    import paged_kv_decode_attn_amd as pkd
    lens = (40, 50, 70, 100, 33, 64, 65, 129, 97)
    w = wl.make("attn", "cpu", seed=31 + nq + d + kvt, n_q=nq, n_kv=nkv, d=d, kv_dtype=kvt, lens=lens,
                append=append, chunk=8, shared_first_page=True)
    tables = w.tables.copy()
    used = {int(tables[s][j]) for s in range(len(lens)) for j in range(int(w.counts[s]))}
    free = sorted(set(range(w.num_pages)) - used)
    k = 0
    for s in range(1, len(lens)):
        if tables[s][0] == tables[0][0]:
            tables[s][0] = free[k]
            k += 1
    assert k >= 2
    w_private = dataclasses.replace(w, tables=tables)
    pool_shared, pool_private = H.GpuPool(w), H.GpuPool(w_private)
    assert pkd.pkd_pool_info_get(pool_shared.handle).shared_pages == 1
    assert pkd.pkd_pool_info_get(pool_private.handle).shared_pages == 0
    dev = lambda t: None if t is None else t.to("cuda")
    outs = [H.run_attention(pool, w.seq, w.pos, dev(w.q), dev(w.k_new), dev(w.v_new), wl.F32,
                            distinct=True).cpu() for pool in (pool_shared, pool_private)]
    assert torch.equal(outs[0], outs[1])


PREFILL_CASES = [
    # (kv dtype, q heads, kv heads, head dim, chunk pages).  A tile has 128 columns
    # (64 for f32 pools) of (row, query head) pairs: rows per tile = the largest
    # power of two with rows x G within that
    (wl.BF16, 4, 2, 128, 2),    # G 2: tiles of 64 rows
    (wl.BF16, 28, 4, 128, 8),   # G 7: tiles of 16 rows (112 columns)
    (wl.FP8, 16, 8, 128, 3),    # G 2, fp8 pool
    (wl.F32, 4, 2, 64, 2),      # f32 pool: tiles of 32 rows
    (wl.BF16, 16, 1, 64, 5),    # G 16: tiles of 8 rows
]


@pytest.mark.parametrize("kvt,nq,nkv,d,chunk", PREFILL_CASES)
def test_prefill_tiles_bit_identical(H, orc, kvt, nq, nkv, d, chunk):
    """A prompt slice (consecutive positions of one sequence) between decode
    rows of other sequences: its rows are read as shared tiles, each K/V page
    fetched once per tile into LDS.  Outputs are bit-identical to the per-row kernels (the same
    rows afterwards, tiles off) and match the oracle; the slice starts and
    ends off the tile grid."""
    import paged_kv_decode_attn_amd as pkd
    lens = (1100, 40, 200, 33)
    w = wl.make("attn", "cpu", seed=11, n_q=nq, n_kv=nkv, d=d, kv_dtype=kvt, lens=lens, append=True, chunk=chunk,
                extra_pages=6)
    gen = torch.Generator().manual_seed(12)
    qd = wl.F32 if kvt == wl.F32 else wl.BF16
    # 150 slice rows at positions 1001.. (tiles need a 128-row call and a last position >= 1024)
    n_slice = 150
    seq = np.concatenate([[1, 2], np.zeros(n_slice, np.int32), [3]]).astype(np.int32)
    pos = np.concatenate([[39, 199], np.arange(1001, 1001 + n_slice), [32]]).astype(np.int32)
    n = seq.size
    q = wl.encode(torch.randn((n, nq, d), generator=gen), qd)
    kn = wl.encode(torch.randn((n, nkv, d), generator=gen), qd)
    vn = wl.encode(torch.randn((n, nkv, d), generator=gen), qd)
    pool = H.GpuPool(w)
    out = H.run_attention(pool, seq, pos, q.cuda(), kn.cuda(), vn.cuda()).cpu()
    pkd.pkd_pool_check(pool.handle)
    # tiles off: the same rows through the per-row kernels, reading the tokens appended above
    ref = H.run_attention(pool, seq, pos, q.cuda(), None, None, distinct=True).cpu()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    want = oracle_attn(orc, w, seq, pos, q, kn, vn)
    e = H.rel_err(out.numpy(), want)
    print(f"prefill tiles kv{kvt} G{nq // nkv} d{d} chunk {chunk}: {e:.2e}")
    assert e <= TOL_F32_OUT


@pytest.mark.parametrize("chunk", [2, 5])
def test_prefill_tile_invalid_rows(H, chunk):
    """A shared tile whose last rows run past the pages set for the sequence:
    those rows are zeroed and reported, the others keep their bits."""
    import paged_kv_decode_attn_amd as pkd
    w = wl.make("attn", "cpu", seed=13, n_q=4, n_kv=2, d=128, kv_dtype=wl.BF16, lens=(1100,), append=True,
                chunk=chunk, extra_pages=0)
    gen = torch.Generator().manual_seed(14)
    cap = 32 * int(w.counts[0])  # positions the table covers
    n = 128
    p0 = cap - 122
    seq = np.zeros(n, np.int32)
    pos = np.arange(p0, p0 + n, dtype=np.int32)  # the last 6 rows are past the table
    q = wl.encode(torch.randn((n, 4, 128), generator=gen), wl.BF16).cuda()
    kn = wl.encode(torch.randn((n, 2, 128), generator=gen), wl.BF16).cuda()
    vn = wl.encode(torch.randn((n, 2, 128), generator=gen), wl.BF16).cuda()
    pool = H.GpuPool(w)
    out = H.run_attention(pool, seq, pos, q, kn, vn).cpu()
    with pytest.raises(pkd.PkdError) as ei:
        pkd.pkd_pool_check(pool.handle)
    assert ei.value.needed & 2
    assert (out[122:].view(torch.int16) == 0).all()
    ref = H.run_attention(pool, seq[:122], pos[:122], q[:122].contiguous(), None, None, distinct=True).cpu()
    assert torch.equal(out[:122].view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("kvt,chunk", [(wl.BF16, 2), (wl.BF16, 100), (wl.FP8, 3), (wl.F32, 100)])
def test_full_tables(H, orc, kvt, chunk):
    """Rows whose token lands in the last slot of the last page their table
    holds (no spare pages): the largest position a table admits, with and
    without the append fused."""
    lens = (32, 64, 96, 320)
    w = wl.make("attn", "cpu", seed=21 + kvt + chunk, n_q=8, n_kv=2, d=128, kv_dtype=kvt, lens=lens, append=True,
                chunk=chunk, extra_pages=0)
    assert all(int(w.pos[s]) == 32 * int(w.counts[s]) - 1 for s in range(len(lens)))
    want = oracle_attn(orc, w, w.seq, w.pos, w.q, w.k_new, w.v_new)
    for distinct in (False, True):
        pool = H.GpuPool(w)
        out = H.run_attention(pool, w.seq, w.pos, w.q.cuda(), w.k_new.cuda(), w.v_new.cuda(), wl.F32, distinct)
        import paged_kv_decode_attn_amd as pkd
        pkd.pkd_pool_check(pool.handle)
        e = H.rel_err(out.cpu().numpy(), want)
        print(f"full tables kv{kvt} chunk {chunk} distinct={distinct}: {e:.2e}")
        assert e <= TOL_F32_OUT


@pytest.mark.parametrize("chunk", [100, 80])
def test_fused_append_long_rows(H, orc, chunk):
    """The fused append for rows whose own page lies 64 or more pages past the
    start of the wave's page range (2,100- and 2,600-token contexts): outputs
    and pool bytes equal the separate append's, and the oracle's."""
    import paged_kv_decode_attn_amd as pkd
    lens = (2600, 33, 2100)
    w = wl.make("attn", "cpu", seed=77, n_q=4, n_kv=2, d=128, kv_dtype=wl.BF16, lens=lens, append=True,
                chunk=chunk, extra_pages=0)
    outs, pools = [], []
    for distinct in (False, True):
        pool = H.GpuPool(w)
        outs.append(H.run_attention(pool, w.seq, w.pos, w.q.cuda(), w.k_new.cuda(), w.v_new.cuda(), wl.F32,
                                    distinct=distinct).cpu())
        pkd.pkd_pool_check(pool.handle)
        pools.append(pool.pages_bytes().cpu())
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    assert torch.equal(pools[0], pools[1])
    want = oracle_attn(orc, w, w.seq, w.pos, w.q, w.k_new, w.v_new)
    assert H.rel_err(outs[1].numpy(), want) <= TOL_F32_OUT


def _random_attention_cases(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kvt = int(rng.choice([wl.F32, wl.BF16, wl.FP8], p=[0.2, 0.5, 0.3]))
        d = int(rng.choice([64, 128]))
        nkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 7, 8, 16]))
        n_seq = int(rng.integers(1, 6))
        lens = tuple(int(v) for v in rng.choice([1, 2, 31, 32, 33, 200, 700, 2100, 2900], size=n_seq))
        chunk = int(rng.choice([1, 2, 3, 8, 64, 100]))
        extra = int(rng.integers(0, 3))
        cases.append((i, kvt, d, nkv, G, lens, chunk, extra))
    return cases


@pytest.mark.parametrize("i,kvt,d,nkv,G,lens,chunk,extra", _random_attention_cases())
def test_attention_randomized(H, orc, i, kvt, d, nkv, G, lens, chunk, extra):
    """Seeded random geometries (dtype, head dim, GQA group, context lengths up
    to 2,900 tokens, page chunk, spare pages): oracle parity with the append,
    the fused append bit-identical to the separate one, and a shuffled batch
    bit-identical row by row."""
    import paged_kv_decode_attn_amd as pkd
    w = wl.make("attn", "cpu", seed=500 + i, n_q=G * nkv, n_kv=nkv, d=d, kv_dtype=kvt, lens=lens, append=True,
                chunk=chunk, extra_pages=extra)
    print(f"case {i}: kv{kvt} d{d} G{G} n_kv{nkv} lens={lens} chunk={chunk} extra={extra}", flush=True)
    outs, pools = [], []
    for distinct in (False, True):
        pool = H.GpuPool(w)
        outs.append(H.run_attention(pool, w.seq, w.pos, w.q.cuda(), w.k_new.cuda(), w.v_new.cuda(), wl.F32,
                                    distinct=distinct).cpu())
        pkd.pkd_pool_check(pool.handle)
        pools.append(pool.pages_bytes().cpu())
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    assert torch.equal(pools[0], pools[1])
    want = oracle_attn(orc, w, w.seq, w.pos, w.q, w.k_new, w.v_new)
    e = H.rel_err(outs[0].numpy(), want)
    assert e <= TOL_F32_OUT, e
    perm = np.random.default_rng(i).permutation(w.n_rows)
    pool = H.GpuPool(w)
    sh = H.run_attention(pool, w.seq[perm], w.pos[perm], w.q[perm].cuda(), w.k_new[perm].cuda(),
                         w.v_new[perm].cuda(), wl.F32, distinct=True).cpu()
    assert torch.equal(sh.view(torch.int32), outs[0][torch.as_tensor(perm)].view(torch.int32))


def _random_tile_cases(n=6, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kvt = int(rng.choice([wl.F32, wl.BF16, wl.FP8]))
        d = int(rng.choice([64, 128]))
        nkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 5, 7, 16]))
        chunk = int(rng.choice([1, 2, 5, 8, 16]))
        p0 = int(rng.integers(1000, 2200))
        n_slice = int(rng.integers(128, 260))
        lead = int(rng.integers(0, 5))  # decode rows before the slice (shifts it off the tile grid)
        out.append((i, kvt, d, nkv, G, chunk, p0, n_slice, lead))
    return out


@pytest.mark.parametrize("i,kvt,d,nkv,G,chunk,p0,n_slice,lead", _random_tile_cases())
def test_prefill_tiles_randomized(H, orc, i, kvt, d, nkv, G, chunk, p0, n_slice, lead):
    """Seeded random prompt slices read as shared tiles (odd G, every pool
    dtype, random chunk sizes and offsets): bit-identical to the per-row
    kernels and within the oracle's tolerance."""
    lens = (p0 + n_slice + 40,) + tuple(range(40, 40 + 30 * lead, 30))
    w = wl.make("attn", "cpu", seed=900 + i, n_q=G * nkv, n_kv=nkv, d=d, kv_dtype=kvt, lens=lens, append=True,
                chunk=chunk, extra_pages=1)
    gen = torch.Generator().manual_seed(901 + i)
    qd = wl.F32 if kvt == wl.F32 else wl.BF16
    seq = np.concatenate([np.arange(1, 1 + lead), np.zeros(n_slice)]).astype(np.int32)
    pos = np.concatenate([np.asarray(lens[1:], np.int32) - 1, np.arange(p0, p0 + n_slice)]).astype(np.int32)
    n = seq.size
    q = wl.encode(torch.randn((n, G * nkv, d), generator=gen), qd)
    kn = wl.encode(torch.randn((n, nkv, d), generator=gen), qd)
    vn = wl.encode(torch.randn((n, nkv, d), generator=gen), qd)
    print(f"tiles case {i}: kv{kvt} d{d} G{G} n_kv{nkv} chunk {chunk} slice {p0}+{n_slice} lead {lead}", flush=True)
    pool = H.GpuPool(w)
    out = H.run_attention(pool, seq, pos, q.cuda(), kn.cuda(), vn.cuda()).cpu()
    ref = H.run_attention(pool, seq, pos, q.cuda(), None, None, distinct=True).cpu()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    want = oracle_attn(orc, w, seq, pos, q, kn, vn)
    assert H.rel_err(out.numpy(), want) <= TOL_F32_OUT


def _decode_codes(codes: torch.Tensor, kvt: int, scale: float) -> torch.Tensor:
    if kvt == wl.F32:
        return codes.float()
    if kvt == wl.BF16:
        return codes.view(torch.bfloat16).float()
    return codes.view(torch.float8_e4m3fn).float() * scale


@pytest.mark.parametrize("kvt,chunk", [(wl.BF16, 2), (wl.BF16, 100), (wl.FP8, 3), (wl.F32, 5)])
def test_reference_moves_mid_row(H, orc, kvt, chunk):
    """Keys planted in later pages score far above every earlier key (base-2
    jumps of about 14, 28, 56 and 112, against the softmax reference's slack
    of 8), so the reference moves and O and l are rescaled in the middle of a
    row, which random keys almost never make happen.  Per-row kernels and
    shared tiles against the oracle, tiles bit-identical to the per-row
    kernels (chunk 100 leaves the pool unchunked: the direct kernel)."""
    import paged_kv_decode_attn_amd as pkd
    nq, nkv, d = 8, 2, 128
    lens = (1300, 300, 700)
    w = wl.make("attn", "cpu", seed=31, n_q=nq, n_kv=nkv, d=d, kv_dtype=kvt, lens=lens, append=False,
                chunk=chunk, extra_pages=0)
    gen = torch.Generator().manual_seed(32)
    c = torch.randn(d, generator=gen)
    c = c / c.norm()
    qd = wl.F32 if kvt == wl.F32 else wl.BF16

    def queries(n):  # every query leans on c (q . c ~ 11 +- 1), so keys along c score high for all
        return wl.encode(torch.randn((n, nq, d), generator=gen) + 11.0 * c, qd)

    hk = _decode_codes(w.hist_k, kvt, w.k_scale).clone()
    for s, L in enumerate(w.hist_len):
        o = int(w.hist_off[s])
        for t, beta in ((100, 10.0), (260, 20.0), (650, 40.0), (1210, 80.0)):
            if t < L:
                hk[o + t] = beta * c
    ks = wl.fp8_scale(hk) if kvt == wl.FP8 else 1.0
    w.hist_k = wl.encode(hk, kvt, ks)
    w.k_scale = ks
    w.q = queries(len(lens))
    pool = H.GpuPool(w)
    out = H.run_attention(pool, w.seq, w.pos, w.q.cuda(), None, None, distinct=True).cpu()
    e = H.rel_err(out.numpy(), oracle_attn(orc, w, w.seq, w.pos, w.q))
    print(f"reference moves, kv{kvt} chunk {chunk}: per row {e:.2e}", flush=True)
    assert e <= TOL_F32_OUT
    # a 200-row prompt slice of sequence 0 at positions 1000..1199
    n = 200
    seq = np.zeros(n, np.int32)
    pos = np.arange(1000, 1000 + n, dtype=np.int32)
    q2 = queries(n)
    tiled = H.run_attention(pool, seq, pos, q2.cuda(), None, None).cpu()
    per_row = H.run_attention(pool, seq, pos, q2.cuda(), None, None, distinct=True).cpu()
    assert torch.equal(tiled.view(torch.int32), per_row.view(torch.int32))
    e2 = H.rel_err(tiled.numpy(), oracle_attn(orc, w, seq, pos, q2))
    print(f"  slice {e2:.2e}", flush=True)
    assert e2 <= TOL_F32_OUT
    pkd.pkd_pool_check(pool.handle)
