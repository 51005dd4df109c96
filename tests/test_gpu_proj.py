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
    (wl.FP8, wl.BF16, 300, 3584, 2, False, False, wl.F32),
    (wl.FP8, wl.F32, 2 * 64, 1024, 9, True, False, wl.BF16),
    # enough row groups (>= 8192) that K is not split across a block's waves
    (wl.BF16, wl.BF16, 33000, 256, 3, False, True, wl.F32),
    (wl.BF16, wl.BF16, 2 * 16400, 256, 16, True, False, wl.BF16),
    (wl.FP8, wl.BF16, 32768, 256, 5, False, False, wl.F32),
]


@pytest.mark.parametrize("wdt,xdt,rows,cols,n,silu,res,out", GEMV_CASES)
def test_gemv_parity(H, orc, wdt, xdt, rows, cols, n, silu, res, out):
    seed = rows + cols + n
    W, s = make_w(rows, cols, wdt, seed)
    x = make_x(n, cols, xdt, seed)
    residual = torch.randn((n, rows)) if res else None
    y, yb = run_proj(H, W, rows, cols, wdt, s, 0, x, xdt, n, out, silu, residual, y2=True)
    want = oracle_proj(orc, W, wdt, s, x, xdt, 0, silu, residual)
    got = H.values(y, out)
    e = H.rel_err(got, want)
    print(f"gemv w{wdt} x{xdt} {rows}x{cols} n={n} silu={silu}: {e:.2e}")
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


def test_mfma_tile_height_invariance(H):
    """A large batch runs on the 256-row activation tile and a small one on the
    128-row tile; a row's outputs are bit-identical either way."""
    rows, cols = 16384, 512
    W, s = make_w(rows, cols, wl.BF16, 11)
    x = make_x(1100, cols, wl.BF16, 12)
    full, _ = run_proj(H, W, rows, cols, wl.BF16, 1.0, 1, x, wl.BF16, 1100, wl.F32)
    full = full.cpu()
    for r, n in [(0, 3), (255, 2), (1097, 3), (600, 40)]:
        part, _ = run_proj(H, W, rows, cols, wl.BF16, 1.0, 1, x[r:r + n], wl.BF16, n, wl.F32)
        assert torch.equal(part.cpu(), full[r:r + n]), (r, n)


@pytest.mark.parametrize("family,rows", [(0, 256), (0, 33000), (1, 256)])
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
