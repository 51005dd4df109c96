"""Parity of the projections (vector-ALU GEMV family and matrix-core family,
bf16 / f32 / fp8 weights) against the oracle's fp64 matvec, and batch
invariance of each family."""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

# fp32 accumulation over K <= 18944 terms against fp64: relative error of the
# order sqrt(K) * 2^-24 ~ 1e-5 at worst; 1e-4 is the gate for f32 outputs,
# plus one bf16 rounding (2^-8) for bf16 outputs.
TOL = 1e-4
TOL_BF16 = 2 ** -8 + 1e-4


@pytest.fixture(scope="module")
def H():
    import gpu_harness
    return gpu_harness


def make_w(rows, cols, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    v = torch.randn((rows, cols), generator=g) * 0.02
    s = wl.fp8_scale(v) if dtype == wl.FP8 else 1.0
    return wl.encode(v, dtype, s), s


def make_x(n, cols, dtype, seed):
    g = torch.Generator().manual_seed(seed + 1000)
    v = torch.randn((n, cols), generator=g)
    return wl.encode(v, dtype) if dtype == wl.BF16 else v


def oracle_proj(orc, W, wdt, s, x, xdt, family, silu=False, residual=None):
    Wn = wl.to_numpy_codes(W, wdt)
    xv = (orc.bf16_value(wl.to_numpy_codes(x, wl.BF16)) if xdt == wl.BF16 else
          x.numpy().astype(np.float64))
    if family == 1 and wdt == wl.FP8:
        rows = []
        for r in range(xv.shape[0]):
            codes, sz = orc.act_quant(xv[r])
            rows.append((orc.e4m3_value(codes), sz))
        y = np.stack([orc.matvec_rows(wdt, Wn, s, c[None])[0] * sz for c, sz in rows])
    else:
        y = orc.matvec_rows(wdt, Wn, s, xv)
    if silu:
        F = y.shape[1] // 2
        g, u = y[:, :F], y[:, F:]
        y = g / (1 + np.exp(-g)) * u
    if residual is not None:
        y = y + residual.numpy().astype(np.float64)
    return y


def run_proj(H, W, rows, cols, wdt, s, family, x, xdt, n, out_dtype, silu=False, residual=None, y2=False,
             k_splits=1):
    import paged_kv_decode_attn_amd as pkd
    Wd = W.cuda()
    M = pkd.make_matrix(Wd, rows, cols, wdt, s, family, k_splits)
    nout = rows // 2 if silu else rows
    y = torch.empty((n, nout), dtype=torch.float32 if out_dtype == wl.F32 else torch.int16, device="cuda")
    yb = torch.empty((n, nout), dtype=torch.int16, device="cuda") if y2 else None
    wsb = pkd.pkd_gemv_workspace_bytes(M, n)
    ws = H.aligned_empty(wsb) if wsb else None
    pkd.gemv_rows(M, x.cuda(), xdt, n, y, out_dtype, None if residual is None else residual.cuda(), silu, yb, ws)
    torch.cuda.synchronize()
    return y, yb


GEMV_CASES = [
    # (w dtype, x dtype, rows, cols, n rows, silu, residual, out)
    (wl.BF16, wl.BF16, 1000, 3584, 1, False, False, wl.F32),
    (wl.BF16, wl.BF16, 256, 1024, 3, False, True, wl.F32),
    (wl.BF16, wl.F32, 130, 512, 8, False, False, wl.BF16),
    (wl.BF16, wl.BF16, 2 * 192, 1024, 16, True, False, wl.BF16),
    (wl.BF16, wl.BF16, 260, 18944, 5, False, True, wl.F32),
    (wl.F32, wl.F32, 512, 256, 4, False, False, wl.F32),
    (wl.F32, wl.F32, 256, 256, 37, False, True, wl.F32),
    # f32 weights against bf16 activations (4-element activation vectors)
    (wl.F32, wl.BF16, 9000, 3584, 3, True, False, wl.F32),
    (wl.F32, wl.BF16, 700, 192, 17, False, True, wl.BF16),
    (wl.FP8, wl.BF16, 300, 3584, 2, False, False, wl.F32),
    (wl.FP8, wl.F32, 2 * 64, 1024, 9, True, False, wl.BF16),
    # enough row groups (>= 8192) that K is not split across a block's waves
    (wl.BF16, wl.BF16, 33000, 256, 3, False, True, wl.F32),
    (wl.BF16, wl.BF16, 2 * 16400, 256, 16, True, False, wl.BF16),
    (wl.FP8, wl.BF16, 32768, 256, 5, False, False, wl.F32),
]


GEMV_FAMILY_CASES = [(0,) + c for c in GEMV_CASES] + [
    (3,) + c for c in GEMV_CASES if c[1] == wl.BF16 and c[0] != wl.F32] + [
    (3, wl.BF16, wl.BF16, 1000, 3584, 37, False, True, wl.F32),  # three 16-row activation tiles, ragged
    (3, wl.FP8, wl.BF16, 2 * 520, 1024, 20, True, False, wl.BF16),
    # 4,096+ row groups: one wave per K range, two row groups per wave (odd count)
    (3, wl.BF16, wl.BF16, 70000, 256, 17, False, True, wl.F32),
    (3, wl.FP8, wl.BF16, 2 * 33000, 256, 9, True, False, wl.BF16),
]


@pytest.mark.parametrize("fam,wdt,xdt,rows,cols,n,silu,res,out", GEMV_FAMILY_CASES)
def test_gemv_parity(H, orc, fam, wdt, xdt, rows, cols, n, silu, res, out):
    """Vector family (0) and the matrix-core GEMV family (3) against the oracle."""
    seed = rows + cols + n
    W, s = make_w(rows, cols, wdt, seed)
    x = make_x(n, cols, xdt, seed)
    residual = torch.randn((n, rows)) if res else None
    y, yb = run_proj(H, W, rows, cols, wdt, s, fam, x, xdt, n, out, silu, residual, y2=True)
    want = oracle_proj(orc, W, wdt, s, x, xdt, 0, silu, residual)
    got = H.values(y, out)
    e = H.rel_err(got, want)
    print(f"gemv family {fam} w{wdt} x{xdt} {rows}x{cols} n={n} silu={silu}: {e:.2e}")
    assert e <= (TOL if out == wl.F32 else TOL_BF16)
    assert H.rel_err(H.values(yb, wl.BF16), want) <= TOL_BF16


MFMA_CASES = [
    # (family, w dtype, x dtype, rows, cols, n rows, silu, residual, out, k splits)
    (1, wl.BF16, wl.BF16, 256, 256, 1, False, False, wl.F32, 1),
    (1, wl.BF16, wl.BF16, 384, 1024, 130, False, True, wl.F32, 1),
    (1, wl.BF16, wl.BF16, 2 * 192, 512, 257, True, False, wl.BF16, 1),
    (1, wl.BF16, wl.BF16, 128, 3584, 64, False, False, wl.BF16, 1),
    (1, wl.BF16, wl.BF16, 512, 3584, 70, False, True, wl.F32, 3),
    (1, wl.BF16, wl.BF16, 2 * 256, 2048, 90, True, False, wl.BF16, 4),
    (1, wl.FP8, wl.F32, 256, 3584, 200, False, True, wl.F32, 1),
    (1, wl.FP8, wl.BF16, 2 * 128, 1024, 33, True, False, wl.BF16, 1),
    (1, wl.FP8, wl.BF16, 128, 18944, 17, False, False, wl.F32, 6),
    (2, wl.FP8, wl.F32, 256, 3584, 200, False, True, wl.F32, 1),
    (2, wl.FP8, wl.BF16, 2 * 128, 1024, 33, True, False, wl.BF16, 1),
    (2, wl.FP8, wl.BF16, 128, 18944, 17, False, False, wl.F32, 2),
    # enough tiles that the 256-row activation tile is chosen (ragged in rows)
    (1, wl.BF16, wl.BF16, 16384, 512, 1100, False, True, wl.F32, 1),
    (1, wl.BF16, wl.BF16, 2 * 8192, 512, 1030, True, False, wl.BF16, 1),
    (1, wl.BF16, wl.BF16, 2 * 4096, 1024, 513, True, False, wl.BF16, 3),
    (1, wl.FP8, wl.BF16, 16384, 1024, 777, False, False, wl.F32, 1),
    (2, wl.FP8, wl.F32, 8192, 2048, 600, False, True, wl.F32, 4),
    (2, wl.FP8, wl.BF16, 2 * 8192, 1024, 1000, True, False, wl.BF16, 1),
]

# the oracle checks a spread of rows of the big cases (first, last, ragged tail)
def sample_rows(n):
    if n <= 300:
        return np.arange(n)
    g = np.random.default_rng(n)
    return np.unique(np.concatenate([[0, 1, n - 1, n - 2], g.choice(n, 28, replace=False)]))


@pytest.mark.parametrize("fam,wdt,xdt,rows,cols,n,silu,res,out,S", MFMA_CASES)
def test_mfma_parity(H, orc, fam, wdt, xdt, rows, cols, n, silu, res, out, S):
    seed = rows + cols + n + 7
    W, s = make_w(rows, cols, wdt, seed)
    x = make_x(n, cols, xdt, seed)
    residual = torch.randn((n, rows)) if res else None
    y, yb = run_proj(H, W, rows, cols, wdt, s, fam, x, xdt, n, out, silu, residual, y2=True, k_splits=S)
    idx = sample_rows(n)
    want = oracle_proj(orc, W, wdt, s, x[idx], xdt, 1, silu, None if residual is None else residual[idx])
    got = H.values(y, out)[idx]
    e = H.rel_err(got, want)
    print(f"mfma family {fam} w{wdt} x{xdt} {rows}x{cols} n={n} silu={silu} S={S}: {e:.2e}")
    assert e <= (TOL if out == wl.F32 else TOL_BF16)
    if fam == 1 and out == wl.F32:
        assert e <= 2e-6  # products exact and sums fp32-accurate
    assert H.rel_err(H.values(yb, wl.BF16)[idx], want) <= TOL_BF16


@pytest.mark.parametrize("cols,k_splits", [(512, 1), (512, 2), (64, 1), (128, 1), (192, 1), (192, 2), (320, 3)])
def test_mfma_tile_height_invariance(H, cols, k_splits):
    """A large batch runs on the 256-row activation tile (2,048 rows over 64
    weight tiles: two rounds of 256-row tiles against four of 128-row ones) and
    a small one on the 128-row tile; a row's outputs are bit-identical either
    way, with and without a K split, down to K ranges of one to five 64-wide
    k-steps (the first and last stages of the tile's load pipeline)."""
    rows, n_all = 16384, 2048
    W, s = make_w(rows, cols, wl.BF16, 11)
    x = make_x(n_all, cols, wl.BF16, 12)
    full, _ = run_proj(H, W, rows, cols, wl.BF16, 1.0, 1, x, wl.BF16, n_all, wl.F32, k_splits=k_splits)
    full = full.cpu()
    for r, n in [(0, 3), (255, 2), (2045, 3), (600, 40), (1100, 129)]:
        part, _ = run_proj(H, W, rows, cols, wl.BF16, 1.0, 1, x[r:r + n], wl.BF16, n, wl.F32, k_splits=k_splits)
        assert torch.equal(part.cpu(), full[r:r + n]), (r, n)


@pytest.mark.parametrize("family,wdt,k_splits", [(1, wl.BF16, 1), (1, wl.BF16, 3), (2, wl.FP8, 1), (2, wl.FP8, 3)])
def test_mfma_tile_windows_cover_every_tile(H, family, wdt, k_splits):
    """With 8 or more activation tiles the matrix-core tiles run in windows
    of 4 weight units (weight tile x K split) x the activation tiles, the last
    window group shorter when the unit count is not a multiple of 4 (5 weight
    tiles: groups of 4 + 1 units, or 4 + 4 + 4 + 3 with 3 splits).  Every
    output is written (the output starts as NaN) and equals, bit for bit, the
    same rows run in 256-row launches (fewer than 8 activation tiles: the
    plain order)."""
    import paged_kv_decode_attn_amd as pkd
    rows, cols, n_all = 1280, 512, 2048
    W, s = make_w(rows, cols, wdt, 31 + k_splits)
    x = make_x(n_all, cols, wl.BF16, 32)
    M = pkd.make_matrix(W.cuda(), rows, cols, wdt, s, family, k_splits)
    xd = x.cuda()

    def run(r0, n):
        y = torch.full((n, rows), float("nan"), dtype=torch.float32, device="cuda")
        wsb = pkd.pkd_gemv_workspace_bytes(M, n)
        ws = H.aligned_empty(wsb) if wsb else None
        pkd.gemv_rows(M, xd[r0:r0 + n], wl.BF16, n, y, wl.F32, None, False, None, ws)
        torch.cuda.synchronize()
        return y.cpu()

    full = run(0, n_all)
    assert not torch.isnan(full).any()
    for r0 in range(0, n_all, 256):
        assert torch.equal(run(r0, 256), full[r0:r0 + 256]), r0


@pytest.mark.parametrize("family,cols,k_splits,silu", [(2, 512, 1, False), (2, 512, 1, True), (2, 128, 1, True),
                                                     (2, 384, 1, False), (2, 1024, 2, False), (1, 512, 1, True),
                                                     (1, 256, 2, False)])
def test_mfma_fp8_tile_height_invariance(H, family, cols, k_splits, silu):
    """fp8 weights on the matrix cores (native fp8 instruction: family 2; codes
    decoded to bf16: family 1): a large batch runs on the 256-row activation
    tile (the ring pipeline, and the L2 weight prefetch for stacked gate/up
    matrices), a small one on the 128-row tile; a row's outputs are
    bit-identical either way, down to K ranges of one 128-wide fp8 step."""
    rows, n_all = 16384, 2048
    W, s = make_w(rows, cols, wl.FP8, 21 + cols)
    x = make_x(n_all, cols, wl.BF16, 22 + cols)
    full, _ = run_proj(H, W, rows, cols, wl.FP8, s, family, x, wl.BF16, n_all, wl.BF16, silu=silu, k_splits=k_splits)
    full = full.cpu()
    for r, n in [(0, 3), (255, 2), (2045, 3), (600, 40), (1100, 129)]:
        part, _ = run_proj(H, W, rows, cols, wl.FP8, s, family, x[r:r + n], wl.BF16, n, wl.BF16, silu=silu,
                           k_splits=k_splits)
        assert torch.equal(part.cpu(), full[r:r + n]), (r, n)


@pytest.mark.parametrize("family,rows", [(0, 256), (0, 33000), (1, 256), (3, 256), (3, 70000)])
def test_projection_batch_invariance(H, family, rows):
    """A row's outputs are bit-identical alone, in any batch size (the vector
    family's register tile changes with the batch) and at any position; for
    the vector family both with K split over a block's waves (256 rows) and
    without (33000 rows)."""
    cols = 1024
    W, s = make_w(rows, cols, wl.BF16, 1)
    x = make_x(300, cols, wl.BF16, 2)
    full, _ = run_proj(H, W, rows, cols, wl.BF16, 1.0, family, x, wl.BF16, 300, wl.F32)
    full = full.cpu()
    for r, n in [(0, 1), (5, 3), (17, 16), (299, 1), (100, 7)]:
        sub = x[r:r + n]
        part, _ = run_proj(H, W, rows, cols, wl.BF16, 1.0, family, sub, wl.BF16, n, wl.F32)
        assert torch.equal(part.cpu(), full[r:r + n]), (r, n)
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(3))
    sh, _ = run_proj(H, W, rows, cols, wl.BF16, 1.0, family, x[perm].contiguous(), wl.BF16, 300, wl.F32)
    assert torch.equal(sh.cpu(), full[perm])


# ----------------------------------------------------------------------------- gathered rows
GATHER_CASES = [
    # (w dtype, x dtype, rows, cols, n rows, max_cand); rows < 32768: K split over
    # a block's four waves, rows >= 32768: not split (the dense head's choice)
    (wl.BF16, wl.BF16, 5000, 2048, 1, 28),
    (wl.BF16, wl.BF16, 5000, 2048, 37, 28),
    (wl.BF16, wl.F32, 3000, 512, 9, 5),
    (wl.F32, wl.F32, 1000, 256, 6, 13),
    (wl.FP8, wl.BF16, 2000, 1024, 20, 28),
    (wl.FP8, wl.F32, 2000, 1024, 6, 1),
    (wl.BF16, wl.BF16, 40000, 256, 70, 28),
    (wl.FP8, wl.BF16, 33000, 512, 16, 33),
]


def gather_lists(n, rows, max_cand, seed):
    """Trie-shaped candidate lists plus the edge cases: a full list, an empty
    one, a count above max_cand (clamped), indices outside the matrix (NaN),
    repeats and the last row."""
    cand, n_cand = wl.head_candidates(n, rows, max_cand, seed)
    n_cand[0] = max_cand
    cand[0] = np.resize(np.array([rows - 1, 0], np.int32), max_cand)  # repeats, both ends
    if n > 1:
        n_cand[1] = 0
    if n > 2:
        n_cand[2] = max_cand + 5
        cand[2] = np.arange(max_cand, dtype=np.int32) * 7 % rows
    if n > 3 and max_cand >= 3:
        n_cand[3] = 3
        cand[3, :3] = [-1, rows, rows // 2]
    return cand, n_cand


def run_gather(W, rows, cols, wdt, s, x, xdt, n, cand, n_cand, fill=12345.0, fam=0):
    import paged_kv_decode_attn_amd as pkd
    Wd = W.cuda()  # the matrix descriptor holds a raw pointer: keep the tensor alive
    M = pkd.make_matrix(Wd, rows, cols, wdt, s, fam)
    y = torch.full((n, cand.shape[1]), fill, dtype=torch.float32, device="cuda")
    pkd.gemv_gather_rows(M, x.cuda(), xdt, n, torch.from_numpy(cand).cuda(), torch.from_numpy(n_cand).cuda(),
                         cand.shape[1], y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def check_gathered(got, want, dense, cand, n_cand, fill):
    """NaN exactly where the index is bad, the fill where nothing is written,
    the oracle's value within TOL elsewhere, and the dense head's bits."""
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got == fill, want == fill)
    ok = np.isfinite(want) & (want != fill)
    assert ok.any()
    den = np.abs(want[ok]).max()
    e = float(np.abs(got[ok] - want[ok]).max() / den)
    rows = dense.shape[1]
    for r in range(got.shape[0]):
        k = int(min(max(n_cand[r], 0), cand.shape[1]))
        for c in range(k):
            j = cand[r, c]
            if 0 <= j < rows:
                assert got[r, c].tobytes() == np.float64(np.float32(dense[r, j])).tobytes(), (r, c, j)
    return e


GATHER_FAMILY_CASES = [(0,) + c for c in GATHER_CASES] + [
    (3,) + c for c in GATHER_CASES if c[1] == wl.BF16 and c[0] != wl.F32]


@pytest.mark.parametrize("fam,wdt,xdt,rows,cols,n,max_cand", GATHER_FAMILY_CASES)
def test_gather_parity(H, orc, fam, wdt, xdt, rows, cols, n, max_cand):
    """Logits of the listed rows: oracle parity, and bit-identical to the same
    entries of the dense head (gemv_rows over the whole matrix)."""
    seed = rows + cols + n
    W, s = make_w(rows, cols, wdt, seed)
    x = make_x(n, cols, xdt, seed)
    cand, n_cand = gather_lists(n, rows, max_cand, seed)
    fill = 12345.0
    got = run_gather(W, rows, cols, wdt, s, x, xdt, n, cand, n_cand, fill, fam)
    xv = (orc.bf16_value(wl.to_numpy_codes(x, wl.BF16)) if xdt == wl.BF16 else x.numpy().astype(np.float64))
    want = orc.matvec_gathered(wdt, wl.to_numpy_codes(W, wdt), s, xv, cand, n_cand, fill)
    dense, _ = run_proj(H, W, rows, cols, wdt, s, fam, x, xdt, n, wl.F32)
    e = check_gathered(got, want, dense.cpu().numpy(), cand, n_cand, fill)
    print(f"gather family {fam} w{wdt} x{xdt} {rows}x{cols} n={n} max_cand={max_cand}: {e:.2e}")
    assert e <= TOL


@pytest.mark.parametrize("fam", [0, 3])
def test_gather_full_vocabulary_head(H, orc, fam):
    """The tied-embedding head at its full size (151,936 x 2,048 bf16), 64
    rows of up to 28 candidates: every entry bit-identical to the dense head,
    and the oracle on a sample of rows."""
    import paged_kv_decode_attn_amd as pkd
    V, D, C = wl.HEAD_VOCAB, wl.HEAD_HIDDEN, wl.HEAD_MAX_CAND
    n = 64
    g = torch.Generator(device="cuda").manual_seed(77)
    Wd = (torch.randn((V, D), generator=g, device="cuda") * 0.02).to(torch.bfloat16).view(torch.int16)
    x = (torch.randn((n, D), generator=g, device="cuda")).to(torch.bfloat16).view(torch.int16)
    cand, n_cand = wl.head_candidates(n, V, C, 78)
    M = pkd.make_matrix(Wd, V, D, wl.BF16, 1.0, fam)
    y = torch.full((n, C), -5.0, device="cuda")
    pkd.gemv_gather_rows(M, x, wl.BF16, n, torch.from_numpy(cand).cuda(), torch.from_numpy(n_cand).cuda(), C, y)
    dense = torch.empty((n, V), device="cuda")
    pkd.gemv_rows(M, x, wl.BF16, n, dense, wl.F32)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    dn = dense.cpu().numpy()
    for r in range(n):
        k = n_cand[r]
        assert np.array_equal(got[r, :k].view(np.uint32), dn[r, cand[r, :k]].view(np.uint32)), r
        assert (got[r, k:] == -5.0).all()
    rs = [0, 1, 31, n - 1]
    sub = np.unique(cand[rs][cand[rs] >= 0])
    Wsub = Wd[torch.from_numpy(sub).long().cuda()].cpu().numpy().view(np.uint16)
    remap = np.searchsorted(sub, np.where(cand[rs] >= 0, cand[rs], sub[0])).astype(np.int32)
    xv = orc.bf16_value(x[rs].cpu().numpy().view(np.uint16))
    want = orc.matvec_gathered(wl.BF16, Wsub, 1.0, xv, remap, n_cand[rs], -5.0)
    e = H.rel_err(got[rs], want)
    print(f"full head n={n}: {e:.2e}")
    assert e <= TOL


# ----------------------------------------------------------------------------- norm factor, rotary table, epilogue
def test_rms_norm_factor(H, orc):
    """1/rms per row against the oracle (fp32 sum of squares: 1e-6), the bf16
    copy bit-exact (round to nearest even), a row's factor independent of the
    batch, and zero rows give 1/sqrt(eps)."""
    import paged_kv_decode_attn_amd as pkd
    g = torch.Generator().manual_seed(40)
    n, cols = 300, 3584
    x = torch.randn((n, cols), generator=g) * 3.0
    x[7] = 0.0
    xd = x.cuda()
    inv = torch.empty(n, device="cuda")
    xb = torch.empty((n, cols), dtype=torch.int16, device="cuda")
    pkd.rms_norm_factor(xd, n, cols, 1e-6, inv, xb)
    torch.cuda.synchronize()
    want = orc.inv_rms_rows(x.numpy().astype(np.float64), 1e-6)
    got = inv.cpu().numpy().astype(np.float64)
    assert np.abs(got / want - 1).max() < 1e-6
    assert got[7] == np.float32(1 / np.sqrt(np.float32(1e-6)))
    assert torch.equal(xb.cpu(), wl.encode(x, wl.BF16))
    for r0, k in [(0, 1), (5, 3), (299, 1)]:
        part = torch.empty(k, device="cuda")
        pkd.rms_norm_factor(xd[r0:r0 + k].contiguous(), k, cols, 1e-6, part)
        torch.cuda.synchronize()
        assert torch.equal(part.cpu(), inv.cpu()[r0:r0 + k])


def test_rope_table(H):
    """(cos, sin) of pos * base^(-2i/d) within one fp32 rounding of the fp64 values."""
    import paged_kv_decode_attn_amd as pkd
    pos = np.array([0, 1, 31, 32, 1000, 2661, 4095, 70000], np.int32)
    for d, base in [(128, 10000.0), (64, 500000.0)]:
        cs = torch.empty((len(pos), d // 2, 2), device="cuda")
        pkd.rope_table(torch.from_numpy(pos).cuda(), len(pos), d, base, cs)
        torch.cuda.synchronize()
        th = pos[:, None].astype(np.float64) * base ** (-np.arange(d // 2) * 2.0 / d)
        got = cs.cpu().numpy().astype(np.float64)
        assert np.abs(got[..., 0] - np.cos(th)).max() <= 6e-8
        assert np.abs(got[..., 1] - np.sin(th)).max() <= 6e-8
        assert (got[0, :, 0] == 1).all() and (got[0, :, 1] == 0).all()


EPI_CASES = [
    # (family, w dtype, x dtype, rows, cols, n, k splits, silu)
    (0, wl.BF16, wl.BF16, 768, 1024, 5, 1, False),
    (0, wl.F32, wl.F32, 768, 256, 3, 1, False),
    (0, wl.BF16, wl.BF16, 2 * 256, 1024, 9, 1, True),
    (1, wl.BF16, wl.BF16, 768, 1024, 130, 1, False),
    (1, wl.BF16, wl.BF16, 768, 2048, 70, 2, False),
    (1, wl.FP8, wl.BF16, 768, 1024, 33, 1, False),
    (1, wl.BF16, wl.BF16, 2 * 256, 1024, 90, 3, True),
    (2, wl.FP8, wl.F32, 768, 1024, 40, 1, False),
    (3, wl.BF16, wl.BF16, 768, 1024, 21, 1, False),
    (3, wl.FP8, wl.BF16, 2 * 256, 1024, 9, 1, True),
]


@pytest.mark.parametrize("fam,wdt,xdt,rows,cols,n,S,silu", EPI_CASES)
def test_epilogue_row_scale_and_rope(H, orc, fam, wdt, xdt, rows, cols, n, S, silu):
    """Projection epilogue with a per-row factor and (without silu) rotary
    pairs on the first 512 outputs (four heads of 128): against the oracle's
    matvec times the factor, rotated by the oracle's RoPE."""
    import paged_kv_decode_attn_amd as pkd
    seed = rows + cols + n + fam
    W, s = make_w(rows, cols, wdt, seed)
    x = make_x(n, cols, xdt, seed)
    g = torch.Generator().manual_seed(seed + 1)
    rsc = (0.5 + torch.rand(n, generator=g)).float()
    pos = torch.randint(0, 3000, (n,), generator=g, dtype=torch.int32)
    hd, rcols = 128, 0 if silu else 512
    Wd = W.cuda()
    M = pkd.make_matrix(Wd, rows, cols, wdt, s, fam, S)
    cs = torch.empty((n, hd // 2, 2), device="cuda")
    pkd.rope_table(pos.cuda(), n, hd, 10000.0, cs)
    nout = rows // 2 if silu else rows
    y = torch.empty((n, nout), device="cuda")
    wsb = pkd.pkd_gemv_workspace_bytes(M, n)
    pkd.gemv_rows(M, x.cuda(), xdt, n, y, wl.F32, None, silu, None, H.aligned_empty(wsb) if wsb else None,
                  row_scale=rsc.cuda(), rope_cs=None if silu else cs, rope_cols=rcols, rope_head_dim=hd)
    torch.cuda.synchronize()
    if fam == 1 and wdt == wl.FP8 or fam == 2:
        raw = oracle_proj(orc, W, wdt, s, x, xdt, 1)
    else:
        raw = oracle_proj(orc, W, wdt, s, x, xdt, 0)
    raw = raw * rsc.numpy().astype(np.float64)[:, None]
    if silu:
        F = rows // 2
        want = raw[:, :F] / (1 + np.exp(-raw[:, :F])) * raw[:, F:]
    else:
        want = raw.copy()
        want[:, :rcols] = orc.rope_rows(raw[:, :rcols], rcols // hd, hd, pos.numpy(), 10000.0)
    e = H.rel_err(y.cpu().numpy(), want)
    print(f"epilogue fam{fam} w{wdt} {rows}x{cols} n={n} S={S} silu={silu}: {e:.2e}")
    assert e <= TOL


def _random_proj_cases(count=14, seed=314):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        fam = int(rng.choice([0, 1, 2, 3]))
        wdt = int(rng.choice([wl.F32, wl.BF16, wl.FP8]))
        xdt = int(rng.choice([wl.F32, wl.BF16]))
        if fam in (1, 2, 3) and wdt == wl.F32:
            continue
        if fam == 2 and wdt != wl.FP8:
            continue
        if (fam == 3 or (fam == 1 and wdt == wl.BF16)) and xdt != wl.BF16:
            continue
        silu = bool(rng.random() < 0.3)
        rows = int(rng.choice([128, 256, 384, 640, 4096, 9000]))
        if fam in (1, 2):
            rows = (rows + 127) // 128 * 128
        if silu:
            rows = rows // 2 * 2
        cols = int(rng.choice([128, 256, 1024, 2048, 3584]))
        n = int(rng.choice([1, 3, 16, 17, 100, 300]))
        S = int(rng.choice([1, 2, 3])) if fam in (1, 2) else 1
        if fam in (1, 2):
            S = min(S, cols // (128 if fam == 2 else 64))  # at least one K block per split
        res = bool(not silu and rng.random() < 0.4)
        scaled = bool(rng.random() < 0.5)
        rope = bool(not silu and rng.random() < 0.5)
        out.append((len(out), fam, wdt, xdt, rows, cols, n, silu, res, S, scaled, rope))
    return out


@pytest.mark.parametrize("i,fam,wdt,xdt,rows,cols,n,silu,res,S,scaled,rope", _random_proj_cases())
def test_projection_randomized(H, orc, i, fam, wdt, xdt, rows, cols, n, silu, res, S, scaled, rope):
    """Seeded random projections over every family, dtype pair, shape, batch,
    K split and epilogue (residual, silu pair, per-row factor, rotary pairs):
    oracle parity, and the first rows alone give their bits in the batch."""
    import paged_kv_decode_attn_amd as pkd
    seed = 1000 + i
    W, s = make_w(rows, cols, wdt, seed)
    x = make_x(n, cols, xdt, seed)
    g = torch.Generator().manual_seed(seed)
    nout = rows // 2 if silu else rows
    residual = torch.randn((n, rows), generator=g) if res else None
    rsc = (0.5 + torch.rand(n, generator=g)).float() if scaled else None
    hd = 64
    rcols = (nout // hd) * hd if rope else 0
    pos = torch.randint(0, 4000, (n,), generator=g, dtype=torch.int32)
    Wd = W.cuda()
    M = pkd.make_matrix(Wd, rows, cols, wdt, s, fam, S)
    cs = torch.empty((n, hd // 2, 2), device="cuda")
    if rope:
        pkd.rope_table(pos.cuda(), n, hd, 10000.0, cs)
    wsb = pkd.pkd_gemv_workspace_bytes(M, n)
    ws = H.aligned_empty(wsb) if wsb else None
    print(f"proj case {i}: family {fam} w{wdt} x{xdt} {rows}x{cols} n={n} silu={silu} res={res} S={S} "
          f"scaled={scaled} rope={rope}", flush=True)

    def run(m):
        y = torch.empty((m, nout), device="cuda")
        pkd.gemv_rows(M, x[:m].contiguous().cuda(), xdt, m, y, wl.F32,
                      None if residual is None else residual[:m].contiguous().cuda(), silu, None, ws,
                      row_scale=None if rsc is None else rsc[:m].contiguous().cuda(),
                      rope_cs=cs[:m].contiguous() if rope and rcols else None, rope_cols=rcols, rope_head_dim=hd)
        torch.cuda.synchronize()
        return y.cpu()
    y = run(n)
    raw = oracle_proj(orc, W, wdt, s, x, xdt, 1 if (fam in (1, 2) and wdt == wl.FP8) else 0)
    if rsc is not None:
        raw = raw * rsc.numpy().astype(np.float64)[:, None]
    if silu:
        F = rows // 2
        want = raw[:, :F] / (1 + np.exp(-raw[:, :F])) * raw[:, F:]
    else:
        want = raw.copy()
        if rcols:
            want[:, :rcols] = orc.rope_rows(raw[:, :rcols], rcols // hd, hd, pos.numpy(), 10000.0)
        if residual is not None:
            want = want + residual.numpy().astype(np.float64)
    e = H.rel_err(y.numpy(), want)
    print(f"  rel err {e:.2e}", flush=True)
    assert e <= TOL
    m = min(n, 2)
    assert torch.equal(run(m).view(torch.int32), y[:m].view(torch.int32))
