"""The C ABI without a GPU: the library loads, exports every symbol declared in
include/pkd.h, and refuses bad arguments on the host with typed errors and
the numbers involved, before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pkd():
    import paged_kv_decode_attn_amd as p
    if not os.path.exists(p.LIB_PATH):
        from paged_kv_decode_attn_amd import build
        build.build(force=False)
    return p


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pkd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\**([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(pkd):
    names = declared_functions()
    assert len(names) >= 14
    L = ctypes.CDLL(pkd.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(pkd.EXPORTS) == set(names)


def test_version(pkd):
    assert "gfx950" in pkd.pkd_version()


def desc(pkd, **kw):
    d = dict(num_pages=16, page_tokens=32, num_kv_heads=2, head_dim=64, kv_dtype=pkd.F32, k_scale=1.0,
             v_scale=1.0, max_seqs=4, max_pages_per_seq=4, attn_chunk_pages=2)
    d.update(kw)
    return pkd.pkd_pool_desc(**d)


def test_pool_bytes_layout(pkd):
    d = desc(pkd)
    block = 32 * 64 * 4
    pages = 16 * 2 * 2 * block
    want = pages + 256 + 256 + 256  # table (4x4 int32), counts, error word, each 256-aligned
    assert pkd.pkd_pool_bytes(d) == want
    assert pkd.pkd_pool_bytes(desc(pkd, head_dim=96)) == 0
    assert pkd.pkd_pool_bytes(desc(pkd, page_tokens=16)) == 0
    big = desc(pkd, num_pages=131072, num_kv_heads=4, head_dim=128, kv_dtype=pkd.FP8_E4M3, k_scale=0.01,
               v_scale=0.01, max_seqs=4096, max_pages_per_seq=32)
    assert pkd.pkd_pool_bytes(big) == 131072 * 4 * 2 * 32 * 128 + 4096 * 32 * 4 + 4096 * 4 + 256


def _create(pkd, d, nbytes, ptr=1 << 20):
    err = pkd.pkd_error()
    h = ctypes.c_void_p()
    st = pkd.lib().kv_pool_create(ctypes.byref(d), ptr, nbytes, None, ctypes.byref(h), ctypes.byref(err))
    return st, err, h


def test_create_refusals_are_typed(pkd):
    d = desc(pkd)
    need = pkd.pkd_pool_bytes(d)
    st, err, h = _create(pkd, d, need - 1)
    assert st == 3 and err.needed == need and err.available == need - 1 and not h.value
    st, err, h = _create(pkd, desc(pkd, page_tokens=16), 1 << 30)
    assert st == 2 and err.needed == 16 and err.available == 32
    st, err, h = _create(pkd, desc(pkd, head_dim=80), 1 << 30)
    assert st == 2
    st, err, h = _create(pkd, desc(pkd, kv_dtype=pkd.BF16, k_scale=0.5), 1 << 30)
    assert st == 2
    st, err, h = _create(pkd, desc(pkd, kv_dtype=pkd.FP8_E4M3, k_scale=0.0, v_scale=1.0), 1 << 30)
    assert st == 2
    st, err, h = _create(pkd, desc(pkd), 1 << 30, ptr=(1 << 20) + 16)
    assert st == 1  # misaligned buffer
    st, err, h = _create(pkd, desc(pkd, max_seqs=0), 1 << 30)
    assert st == 1


def test_gemv_refusals_are_typed(pkd):
    err = pkd.pkd_error()
    ep = pkd.pkd_epilogue(pkd.F32, None, 0, None)
    W = pkd.pkd_matrix(1 << 20, 64, 100, pkd.BF16, 1.0, pkd.FAMILY_GEMV)
    st = pkd.lib().gemv_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 1, 1 << 21, ctypes.byref(ep), None, 0, None,
                             ctypes.byref(err))
    assert st == 2 and err.needed == 100
    W = pkd.pkd_matrix(1 << 20, 100, 256, pkd.BF16, 1.0, pkd.FAMILY_MFMA)
    st = pkd.lib().gemv_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 4, 1 << 21, ctypes.byref(ep), None, 0, None,
                             ctypes.byref(err))
    assert st == 2  # rows not a multiple of 128 for the matrix-core family
    W = pkd.pkd_matrix(1 << 20, 128, 256, pkd.BF16, 1.0, pkd.FAMILY_MFMA)
    st = pkd.lib().gemv_rows(ctypes.byref(W), 1 << 20, pkd.F32, 4, 1 << 21, ctypes.byref(ep), None, 0, None,
                             ctypes.byref(err))
    assert st == 2  # bf16 matrix-core family needs bf16 activations
    W = pkd.pkd_matrix(1 << 20, 128, 256, pkd.BF16, 0.5, pkd.FAMILY_GEMV)
    st = pkd.lib().gemv_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 4, 1 << 21, ctypes.byref(ep), None, 0, None,
                             ctypes.byref(err))
    assert st == 2  # a scale on bf16 weights
    W = pkd.pkd_matrix(1 << 20, 128, 256, pkd.FP8_E4M3, 0.01, pkd.FAMILY_MFMA)
    assert pkd.pkd_gemv_workspace_bytes(W, 100) == 100 * 256 + 512
    W = pkd.pkd_matrix(1 << 20, 127, 256, pkd.BF16, 1.0, pkd.FAMILY_GEMV)
    ep2 = pkd.pkd_epilogue(pkd.F32, None, 1, None)
    st = pkd.lib().gemv_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 1, 1 << 21, ctypes.byref(ep2), None, 0, None,
                             ctypes.byref(err))
    assert st == 1  # silu pair needs an even row count
    st = pkd.lib().gemv_rows(None, 1 << 20, pkd.BF16, 1, 1 << 21, ctypes.byref(ep), None, 0, None,
                             ctypes.byref(err))
    assert st == 1


def test_null_handles_refused(pkd):
    err = pkd.pkd_error()
    rows = pkd.pkd_rows(None, None, 0)
    assert pkd.lib().paged_attn_decode(None, ctypes.byref(rows), 4, None, None, None, None, 0, None, 0, None,
                                       ctypes.byref(err)) == 1
    assert pkd.lib().decode_step(None, None, ctypes.byref(rows), None, None, None, 0, None,
                                 ctypes.byref(err)) == 1
    assert pkd.lib().block_table_set(None, 0, 1, None, None, None, ctypes.byref(err)) == 1
    assert pkd.lib().pkd_pool_check(None, None, ctypes.byref(err)) == 1


def test_suggested_k_splits(pkd):
    """Host-only split policy: long-K and narrow matrices are split, a wide one
    that already fills the chip is not, the vector family never is."""
    D, F, M = 3584, 18944, 768
    # the measured best S at these 7B shapes (batch 768: qkv 2, W_o 3, gate/up 1,
    # down 6 on 256-row tiles, 115 us against 130 for 3 on 128-row tiles; batch
    # 256: qkv 6 (4 within 5%), down 8)
    assert pkd.pkd_suggest_k_splits(4608, D, 1, M) == 2
    assert pkd.pkd_suggest_k_splits(D, D, 1, M) == 3
    assert pkd.pkd_suggest_k_splits(2 * F, D, 1, M) == 1
    assert pkd.pkd_suggest_k_splits(D, F, 1, M) == 6
    assert pkd.pkd_suggest_k_splits(4608, D, 1, 256) in (4, 6)
    assert pkd.pkd_suggest_k_splits(D, F, 1, 256) == 8
    assert pkd.pkd_suggest_k_splits(D, F, 0, M) == 1
    assert pkd.pkd_suggest_k_splits(D, 1024, 1, M) == 1
    assert pkd.pkd_suggest_k_splits(0, D, 1, M) == 1
    for rows, cols in [(4608, D), (D, F), (2 * F, D)]:
        for m in (1, 64, 768, 4096):
            S = pkd.pkd_suggest_k_splits(rows, cols, 2, m)
            assert S in (1, 2, 3, 4, 6, 8) and (S == 1 or cols // S >= 512)


def test_gather_refusals_are_typed(pkd):
    """Host-side refusals of the candidate-row head, before any launch."""
    err = pkd.pkd_error()
    L = pkd.lib()
    W = pkd.pkd_matrix(1 << 20, 128, 256, pkd.BF16, 1.0, pkd.FAMILY_MFMA)
    assert L.gemv_gather_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 2, 1 << 21, 1 << 22, 4, 1 << 23, None,
                              ctypes.byref(err)) == 2  # matrix-core family
    W = pkd.pkd_matrix(1 << 20, 1000, 256, pkd.BF16, 1.0, pkd.FAMILY_GEMV)
    assert L.gemv_gather_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 70000, 1 << 21, 1 << 22, 4, 1 << 23, None,
                              ctypes.byref(err)) == 2 and err.needed == 70000
    assert L.gemv_gather_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 2, 1 << 21, 1 << 22, 0, 1 << 23, None,
                              ctypes.byref(err)) == 1  # max_cand < 1
    assert L.gemv_gather_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 2, None, 1 << 22, 4, 1 << 23, None,
                              ctypes.byref(err)) == 1  # no candidate list
    assert L.gemv_gather_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 2, (1 << 21) + 2, 1 << 22, 4, 1 << 23, None,
                              ctypes.byref(err)) == 1  # misaligned list
    assert L.gemv_gather_rows(ctypes.byref(W), (1 << 20) + 4, pkd.BF16, 2, 1 << 21, 1 << 22, 4, 1 << 23, None,
                              ctypes.byref(err)) == 1  # misaligned activations
    W = pkd.pkd_matrix(1 << 20, 1000, 100, pkd.BF16, 1.0, pkd.FAMILY_GEMV)
    assert L.gemv_gather_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 2, 1 << 21, 1 << 22, 4, 1 << 23, None,
                              ctypes.byref(err)) == 2  # cols not a multiple of 64
    W = pkd.pkd_matrix(1 << 20, 1000, 256, pkd.BF16, 1.0, pkd.FAMILY_GEMV)
    assert L.gemv_gather_rows(ctypes.byref(W), None, pkd.BF16, 0, None, None, 0, None, None,
                              ctypes.byref(err)) == 0  # nothing to do


def test_norm_rope_refusals_are_typed(pkd):
    """Host-side refusals of the norm factor, the rotary table and the
    epilogue's rotation fields."""
    err = pkd.pkd_error()
    L = pkd.lib()
    assert L.rms_norm_factor(1 << 20, 4, 102, 1e-6, 1 << 21, None, None, ctypes.byref(err)) == 2  # cols % 4
    assert L.rms_norm_factor(1 << 20, 4, 128, -1.0, 1 << 21, None, None, ctypes.byref(err)) == 1  # eps < 0
    assert L.rms_norm_factor(None, 4, 128, 1e-6, 1 << 21, None, None, ctypes.byref(err)) == 1
    assert L.rms_norm_factor((1 << 20) + 4, 4, 128, 1e-6, 1 << 21, None, None, ctypes.byref(err)) == 1
    assert L.rms_norm_factor(None, 0, 128, 1e-6, None, None, None, ctypes.byref(err)) == 0
    assert L.rope_table(1 << 20, 4, 127, 10000.0, 1 << 21, None, ctypes.byref(err)) == 1  # odd head_dim
    assert L.rope_table(1 << 20, 4, 128, 0.0, 1 << 21, None, ctypes.byref(err)) == 1  # base
    assert L.rope_table(None, 4, 128, 10000.0, 1 << 21, None, ctypes.byref(err)) == 1
    assert L.rope_table(None, 0, 128, 10000.0, None, None, ctypes.byref(err)) == 0
    W = pkd.pkd_matrix(1 << 20, 512, 256, pkd.BF16, 1.0, pkd.FAMILY_GEMV)
    for rope_cols, hd, silu in [(512, 126, 0), (384, 256, 0), (1024, 128, 0), (256, 128, 1)]:
        ep = pkd.pkd_epilogue(pkd.F32, None, silu, None, None, 1 << 22, rope_cols, hd)
        st = L.gemv_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 1, 1 << 21, ctypes.byref(ep), None, 0, None,
                         ctypes.byref(err))
        assert st == 1, (rope_cols, hd, silu)


def test_gemv_mfma_family_refusals(pkd):
    """The matrix-core GEMV family takes bf16 or fp8 weights and bf16 activations only."""
    err = pkd.pkd_error()
    ep = pkd.pkd_epilogue(pkd.F32, None, 0, None)
    W = pkd.pkd_matrix(1 << 20, 100, 256, pkd.BF16, 1.0, pkd.FAMILY_GEMV_MFMA)
    assert pkd.lib().gemv_rows(ctypes.byref(W), 1 << 20, pkd.F32, 4, 1 << 21, ctypes.byref(ep), None, 0, None,
                               ctypes.byref(err)) == 2
    W = pkd.pkd_matrix(1 << 20, 100, 256, pkd.F32, 1.0, pkd.FAMILY_GEMV_MFMA)
    assert pkd.lib().gemv_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 4, 1 << 21, ctypes.byref(ep), None, 0, None,
                               ctypes.byref(err)) == 2
    W = pkd.pkd_matrix(1 << 20, 100, 256, pkd.BF16, 1.0, 4)
    assert pkd.lib().gemv_rows(ctypes.byref(W), 1 << 20, pkd.BF16, 4, 1 << 21, ctypes.byref(ep), None, 0, None,
                               ctypes.byref(err)) == 1  # no such family
    assert pkd.pkd_gemv_workspace_bytes(pkd.pkd_matrix(1 << 20, 128, 256, pkd.FP8_E4M3, 0.01,
                                                       pkd.FAMILY_GEMV_MFMA), 64) == 0
