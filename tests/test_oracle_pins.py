"""Pins of the fp64 oracle against things other than itself: format
definitions (golden fixtures), library routines (torch conversions, numpy
matmul, torch scaled_dot_product_attention), closed forms and invariants.
CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _val(v):
    return float(v) if not isinstance(v, str) else float(v.replace("inf", "inf"))


# ----------------------------------------------------------------------------- codecs
def test_bf16_golden(orc):
    g = json.load(open(os.path.join(GOLD, "bf16_points.json")))
    for code, v in g["decode"]:
        got = orc.bf16_value([int(code, 16)])[0]
        want = float(v)
        assert (math.isnan(got) and math.isnan(want)) or got == want, (code, got, want)
    for x, code, why in g["encode_rne"]:
        assert int(orc.bf16_round([x])[0]) == int(code, 16), why


def test_e4m3_golden(orc):
    g = json.load(open(os.path.join(GOLD, "e4m3_ocp.json")))
    for code, v in g["decode"]:
        got = orc.e4m3_value([int(code, 16)])[0]
        want = float(v)
        assert (math.isnan(got) and math.isnan(want)) or (got == want and
                                                          math.copysign(1, got) == math.copysign(1, want)), code
    for x, code, why in g["encode_rne_saturating"]:
        assert int(orc.e4m3_round([float(x)])[0]) == int(code, 16), why


def test_bf16_decode_exhaustive_vs_torch(orc):
    codes = np.arange(65536, dtype=np.uint16)
    mine = orc.bf16_value(codes)
    lib = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])


def test_bf16_encode_roundtrip_and_midpoints(orc):
    codes = np.arange(65536, dtype=np.uint16)
    vals = orc.bf16_value(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(orc.bf16_round(vals[fin]), codes[fin])
    # exact midpoints between consecutive positive finite codes tie to the even code
    pos = codes[(codes < 0x7F7F)]
    lo, hi = orc.bf16_value(pos), orc.bf16_value(pos + 1)
    mid = (lo + hi) / 2
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
    assert np.array_equal(orc.bf16_round(mid), want)


def test_bf16_encode_vs_torch_random(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, 200000),
                        rng.standard_normal(50000)]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_round(x.astype(np.float64)), lib)


def test_e4m3_decode_exhaustive_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_value(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])


def test_e4m3_encode_nearest_bruteforce(orc):
    """Against a brute-force search of the nearest representable value (ties
    to the even code), written from the format's value table."""
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.e4m3_value(codes)
    finite = codes[np.isfinite(vals) & (codes < 0x80)]  # non-negative codes 0x00..0x7E
    fv = vals[finite]
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.uniform(0, 470, 20000), rng.uniform(0, 0.05, 20000),
                        (fv[:-1] + fv[1:]) / 2, fv])
    got = orc.e4m3_round(x)
    for xi, gi in zip(x, got):
        d = np.abs(fv - min(xi, 448.0))
        best = finite[d == d.min()]
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert gi == want, (xi, gi, want)
    assert np.array_equal(orc.e4m3_round(-x), got | 0x80)


def test_e4m3_encode_vs_torch_in_range(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * 60.0).clip(-448, 448).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_round(x.astype(np.float64)), lib)


def test_act_quant_definition(orc):
    rng = np.random.default_rng(4)
    z = rng.standard_normal(3584) * 3.0
    codes, s = orc.act_quant(z)
    zf = z.astype(np.float32)
    assert s == np.float32(np.abs(zf).max()) / np.float32(448.0)
    assert orc.e4m3_value(codes[[np.argmax(np.abs(zf))]])[0] == 448.0 * np.sign(zf[np.argmax(np.abs(zf))])
    deq = orc.e4m3_value(codes) * s
    # E4M3 relative half-ulp bound for normals (2^-4), absolute bound for subnormals
    err = np.abs(deq - zf)
    assert np.all(err <= np.maximum(np.abs(zf) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6))
    codes0, s0 = orc.act_quant(np.zeros(64))
    assert s0 == 1.0 and not codes0.any()


# ----------------------------------------------------------------------------- matvec
def test_matvec_closed_forms(orc):
    rng = np.random.default_rng(5)
    cols = 512
    X = rng.standard_normal((3, cols))
    eye = np.eye(cols, dtype=np.float32)
    assert np.array_equal(orc.matvec_rows(orc.F32, eye, 1.0, X), X)
    onehot = np.zeros((4, cols), np.float32)
    idx = [7, 0, 511, 100]
    onehot[np.arange(4), idx] = 1.0
    assert np.array_equal(orc.matvec_rows(orc.F32, onehot, 1.0, X), X[:, idx])
    ones = np.ones((1, cols), np.float32)
    got = orc.matvec_rows(orc.F32, ones, 1.0, X)[:, 0]
    want = np.array([math.fsum(r) for r in X])
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def test_matvec_vs_numpy_all_dtypes(orc):
    rng = np.random.default_rng(6)
    W = torch.from_numpy(rng.standard_normal((96, 256)).astype(np.float32) * 0.02)
    X = rng.standard_normal((5, 256))
    for dt in (orc.F32, orc.BF16, orc.FP8):
        s = wl.fp8_scale(W) if dt == orc.FP8 else 1.0
        codes = wl.to_numpy_codes(wl.encode(W, dt, s), dt)
        Wv = orc.code_values(codes, dt, s)
        want = X @ Wv.T
        got = orc.matvec_rows(dt, codes, s, X)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-14), dt
        # linearity in x is exact up to fp64 rounding
        assert np.allclose(orc.matvec_rows(dt, codes, s, 2.0 * X), 2.0 * got, rtol=0, atol=0)


def test_matvec_gathered_closed_forms(orc):
    """Identity rows pick the activation entries the candidate list names, in
    the list's order; a bad index gives NaN; entries past the (clamped) count
    keep the caller's fill; a repeated index gives the same value twice."""
    rng = np.random.default_rng(11)
    cols = 256
    X = rng.standard_normal((4, cols))
    eye = np.eye(cols, dtype=np.float32)
    cand = np.array([[5, 0, 255, 5, 9, 9],
                     [255, 254, 1, 0, 0, 0],
                     [3, -1, cols, 7, 0, 0],
                     [11, 12, 13, 14, 15, 16]], np.int32)
    n_cand = np.array([6, 3, 4, 99], np.int32)
    Y = orc.matvec_gathered(orc.F32, eye, 1.0, X, cand, n_cand, fill=-7.0)
    assert np.array_equal(Y[0], X[0, [5, 0, 255, 5, 9, 9]])
    assert np.array_equal(Y[1, :3], X[1, [255, 254, 1]]) and (Y[1, 3:] == -7.0).all()
    assert Y[2, 0] == X[2, 3] and np.isnan(Y[2, 1]) and np.isnan(Y[2, 2]) and Y[2, 3] == X[2, 7]
    assert (Y[2, 4:] == -7.0).all()
    assert np.array_equal(Y[3], X[3, 11:17])  # a count above max_cand is clamped
    Y0 = orc.matvec_gathered(orc.F32, eye, 1.0, X, cand, np.array([0, -3, 0, 0], np.int32), fill=2.5)
    assert (Y0 == 2.5).all()


def test_matvec_gathered_vs_numpy_all_dtypes(orc):
    """Each gathered entry is the product of that weight row with that
    activation row (numpy over the decoded weights), for every storage dtype
    and with a per-tensor scale."""
    rng = np.random.default_rng(12)
    W = torch.from_numpy(rng.standard_normal((300, 128)).astype(np.float32) * 0.05)
    X = rng.standard_normal((6, 128))
    cand = rng.integers(0, 300, size=(6, 28)).astype(np.int32)
    n_cand = np.array([28, 1, 0, 17, 28, 5], np.int32)
    for dt in (orc.F32, orc.BF16, orc.FP8):
        s = wl.fp8_scale(W) if dt == orc.FP8 else 1.0
        codes = wl.to_numpy_codes(wl.encode(W, dt, s), dt)
        Wv = orc.code_values(codes, dt, s)
        got = orc.matvec_gathered(dt, codes, s, X, cand, n_cand, fill=np.nan)
        for r in range(6):
            k = n_cand[r]
            want = Wv[cand[r, :k]] @ X[r]
            assert np.allclose(got[r, :k], want, rtol=1e-12, atol=1e-14), (dt, r)
            assert np.isnan(got[r, k:]).all()


# ----------------------------------------------------------------------------- attention
def _hist(orc, ks, vs, dt=0, n_kv=1, d=4):
    return orc.History([np.asarray(k, dtype={0: np.float32, 1: np.uint16, 2: np.uint8}[dt])
                        for k in ks],
                       [np.asarray(v, dtype={0: np.float32, 1: np.uint16, 2: np.uint8}[dt])
                        for v in vs], dt, n_kv, d)


def test_attention_golden_two_tokens(orc):
    g = json.load(open(os.path.join(GOLD, "attn_two_tokens.json")))
    d = g["head_dim"]
    K = np.asarray(g["K"], np.float32).reshape(2, 1, d)
    V = np.asarray(g["V"], np.float32).reshape(2, 1, d)
    h = _hist(orc, [K], [V])
    q = np.asarray(g["q"], np.float32).reshape(1, 1, d)
    out = orc.attention(1, 1, d, orc.F32, 1.0, 1.0, h, [0], [1], orc.F32, q)
    assert np.allclose(out.reshape(-1), g["out"], rtol=1e-6, atol=1e-6)


def _rand_setup(rng, n_q=4, n_kv=2, d=16, lens=(1, 7, 33, 70)):
    K = [rng.standard_normal((L, n_kv, d)).astype(np.float32) for L in lens]
    V = [rng.standard_normal((L, n_kv, d)).astype(np.float32) for L in lens]
    q = rng.standard_normal((len(lens), n_q, d)).astype(np.float32)
    return K, V, q


def test_attention_closed_forms(orc):
    rng = np.random.default_rng(7)
    n_q, n_kv, d = 4, 2, 16
    lens = (1, 7, 33, 70)
    K, V, q = _rand_setup(rng, n_q, n_kv, d, lens)
    seq = np.arange(4)
    pos = np.asarray(lens) - 1
    h = _hist(orc, K, V, 0, n_kv, d)
    out = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, h, seq, pos, orc.F32, q)
    # L = 1: the output is V_0 exactly
    for hh in range(n_q):
        assert np.array_equal(out[0, hh], V[0][0, hh // 2].astype(np.float64))
    # q = 0: uniform weights, the output is the mean of V
    out0 = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, h, seq, pos, orc.F32, np.zeros_like(q))
    for r, L in enumerate(lens):
        for hh in range(n_q):
            want = np.array([math.fsum(V[r][:, hh // 2, c].astype(np.float64)) / L for c in range(d)])
            assert np.allclose(out0[r, hh], want, rtol=1e-13, atol=1e-15)
    # V constant: weights sum to one, the output is that constant
    Vc = [np.full_like(v, 0.3125) for v in V]
    outc = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, _hist(orc, K, Vc, 0, n_kv, d), seq, pos,
                         orc.F32, q)
    assert np.allclose(outc, 0.3125, rtol=1e-14, atol=0)
    # one key far above the others selects its value
    Kd = [k.copy() for k in K]
    Kd[3][:] = 0
    Kd[3][41, :, :] = 60.0
    qd = np.ones_like(q)
    outd = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, _hist(orc, Kd, V, 0, n_kv, d), seq, pos,
                         orc.F32, qd)
    for hh in range(n_q):
        assert np.allclose(outd[3, hh], V[3][41, hh // 2], rtol=1e-12, atol=1e-12)


def test_attention_gqa_mapping(orc):
    """kv head g carries V = g + 1 everywhere, so q head h must return h // G + 1."""
    rng = np.random.default_rng(8)
    n_q, n_kv, d = 14, 2, 16
    K, _, q = _rand_setup(rng, n_q, n_kv, d, (40,))
    V = [np.broadcast_to(np.arange(1, n_kv + 1, dtype=np.float32)[None, :, None], (40, n_kv, d)).copy()]
    out = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, _hist(orc, K, V, 0, n_kv, d), [0], [39],
                        orc.F32, q)
    for hh in range(n_q):
        assert np.allclose(out[0, hh], hh // 7 + 1, rtol=1e-14, atol=0)


def test_attention_vs_torch_sdpa(orc):
    rng = np.random.default_rng(9)
    n_q, n_kv, d = 8, 2, 64
    lens = (3, 31, 32, 33, 65)
    K, V, q = _rand_setup(rng, n_q, n_kv, d, lens)
    pos = np.asarray(lens) - 1
    out = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, _hist(orc, K, V, 0, n_kv, d),
                        np.arange(len(lens)), pos, orc.F32, q)
    for r, L in enumerate(lens):
        qt = torch.from_numpy(q[r].astype(np.float64))[:, None, :]        # [H, 1, d]
        kt = torch.from_numpy(K[r].astype(np.float64)).permute(1, 0, 2)   # [Hkv, L, d]
        vt = torch.from_numpy(V[r].astype(np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(n_q // n_kv, 0)
        vt = vt.repeat_interleave(n_q // n_kv, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0, :].numpy()
        assert np.allclose(out[r], ref, rtol=1e-11, atol=1e-12), r


def test_attention_extent_and_append_order(orc):
    """A row at position p sees positions 0..p only; rows of one sequence in one
    call see each other's appended tokens exactly as if run one after another."""
    rng = np.random.default_rng(10)
    n_q, n_kv, d = 4, 2, 16
    K, V, q = _rand_setup(rng, n_q, n_kv, d, (50,))
    h = _hist(orc, K, V, 0, n_kv, d)
    full = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, h, [0], [20], orc.F32, q)
    cut = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0,
                        _hist(orc, [K[0][:21]], [V[0][:21]], 0, n_kv, d), [0], [20], orc.F32, q)
    assert np.array_equal(full, cut)
    # three new tokens of one sequence appended and attended in one call ...
    base_k, base_v = K[0][:30], V[0][:30]
    kn = rng.standard_normal((3, n_kv, d)).astype(np.float32)
    vn = rng.standard_normal((3, n_kv, d)).astype(np.float32)
    qn = rng.standard_normal((3, n_q, d)).astype(np.float32)
    hb = _hist(orc, [base_k], [base_v], 0, n_kv, d)
    one = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, hb, [0, 0, 0], [30, 31, 32], orc.F32, qn,
                        kn, vn)
    # ... equal three calls that each append one token onto the grown history
    for j in range(3):
        hj = _hist(orc, [np.concatenate([base_k, kn[:j]])], [np.concatenate([base_v, vn[:j]])], 0,
                   n_kv, d)
        r = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, hj, [0], [30 + j], orc.F32, qn[j:j + 1],
                          kn[j:j + 1], vn[j:j + 1])
        assert np.array_equal(r[0], one[j])


def test_attention_rows_independent(orc):
    rng = np.random.default_rng(11)
    n_q, n_kv, d = 4, 2, 16
    lens = (9, 40, 64, 65, 100)
    K, V, q = _rand_setup(rng, n_q, n_kv, d, lens)
    h = _hist(orc, K, V, 0, n_kv, d)
    pos = np.asarray(lens) - 1
    seq = np.arange(5)
    full = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, h, seq, pos, orc.F32, q)
    perm = np.asarray([3, 0, 4, 2, 1])
    shuf = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, h, seq[perm], pos[perm], orc.F32, q[perm])
    assert np.array_equal(shuf, full[perm])
    alone = orc.attention(n_q, n_kv, d, orc.F32, 1.0, 1.0, h, seq[2:3], pos[2:3], orc.F32, q[2:3])
    assert np.array_equal(alone[0], full[2])


@pytest.mark.parametrize("kv_dtype", [0, 1, 2])
def test_paged_gather_equals_contiguous(orc, kv_dtype):
    """Histories written into a pool at random, reversed and shared pages and
    read back through the block tables equal the contiguous histories bitwise,
    and give bitwise-identical attention."""
    rng = np.random.default_rng(12 + kv_dtype)
    n_kv, d, n_q = 2, 64, 4
    lens = np.asarray([1, 31, 32, 33, 64, 65, 97], np.int32)
    S = len(lens)
    num_pages = 40
    npg = (lens + 31) // 32
    perm = rng.permutation(num_pages)
    lists, o = [], 0
    for i, n in enumerate(npg):
        lists.append(perm[o:o + n].tolist()); o += n
    lists[5] = lists[5][::-1]                     # pages in reverse physical order
    lists[6] = [lists[4][0]] + lists[6][1:]       # first page shared with sequence 4
    tables, counts = wl._finish_tables(lists, S, int(npg.max()))
    gen = torch.Generator().manual_seed(0)
    hk_vals = torch.randn((int(lens.sum()), n_kv, d), generator=gen)
    hv_vals = torch.randn((int(lens.sum()), n_kv, d), generator=gen)
    off = wl._offsets(lens)
    hk_vals[off[6]:off[6] + 32] = hk_vals[off[4]:off[4] + 32]   # shared page content
    hv_vals[off[6]:off[6] + 32] = hv_vals[off[4]:off[4] + 32]
    ks = wl.fp8_scale(hk_vals) if kv_dtype == 2 else 1.0
    vs = wl.fp8_scale(hv_vals) if kv_dtype == 2 else 1.0
    hk, hv = wl.encode(hk_vals, kv_dtype, ks), wl.encode(hv_vals, kv_dtype, vs)
    block = 32 * d * wl.ESIZE[kv_dtype]
    pages = torch.empty(num_pages * n_kv * 2 * block, dtype=torch.uint8)
    wl.fill_pool_pages(pages, num_pages, n_kv, d, kv_dtype, tables, counts, hk, hv, off, lens)
    pages_np = pages.numpy()
    ck, cv = [], []
    for s in range(S):
        k, v = orc.gather_history(pages_np, n_kv, d, kv_dtype, tables[s], int(lens[s]))
        want_k = wl.to_numpy_codes(hk[off[s]:off[s] + lens[s]], kv_dtype)
        want_v = wl.to_numpy_codes(hv[off[s]:off[s] + lens[s]], kv_dtype)
        assert np.array_equal(k.view(np.uint8), want_k.view(np.uint8)), s
        assert np.array_equal(v.view(np.uint8), want_v.view(np.uint8)), s
        ck.append(k); cv.append(v)
    q_dt = 0 if kv_dtype == 0 else 1
    q = wl.to_numpy_codes(wl.encode(torch.randn((S, n_q, d), generator=gen), q_dt), q_dt)
    hist_contig = orc.History([wl.to_numpy_codes(hk[off[s]:off[s] + lens[s]], kv_dtype) for s in range(S)],
                              [wl.to_numpy_codes(hv[off[s]:off[s] + lens[s]], kv_dtype) for s in range(S)],
                              kv_dtype, n_kv, d)
    a = orc.attention(n_q, n_kv, d, kv_dtype, ks, vs, hist_contig, np.arange(S), lens - 1, q_dt, q)
    b = orc.attention(n_q, n_kv, d, kv_dtype, ks, vs, orc.History(ck, cv, kv_dtype, n_kv, d),
                      np.arange(S), lens - 1, q_dt, q)
    assert np.array_equal(a, b)
    # the unset slots of a partial last page read back as the poison bytes
    k0, v0 = orc.gather_history(pages_np, n_kv, d, kv_dtype, tables[0], 32)
    assert (k0[1:].view(np.uint8) == 0xFF).all() and (v0[1:].view(np.uint8) == 0xFF).all()


def test_fp8_append_rounding_is_fp32_division(orc):
    """The row's own value is stored as E4M3(value / scale) with the division in
    fp32 (reading of the fp8 tier).  With value 1.0 and scale fp32(0.84210527)
    the fp32 quotient is exactly 1.1875, a tie that goes to the even code 1.25,
    while the exact quotient 1.18749999... would give 1.125."""
    n_q, n_kv, d = 1, 1, 16
    ks = float(np.float32(0.84210527))
    assert float(np.float32(np.float32(1.0) / np.float32(ks))) == 1.1875
    assert 1.0 / ks < 1.1875
    one = np.full((1, n_kv, d), 0x3F80, np.uint16)  # bf16 1.0
    q = np.zeros((1, n_q, d), np.uint16)
    h = orc.History([np.zeros((0, n_kv, d), np.uint8)], [np.zeros((0, n_kv, d), np.uint8)], 2, n_kv, d)
    out = orc.attention(n_q, n_kv, d, 2, ks, ks, h, [0], [0], 1, q, one, one)
    # with L = 1 the output is the stored value
    assert np.all(out == 1.25 * ks)


# ----------------------------------------------------------------------------- norm and rotary positions
def test_inv_rms_definition(orc):
    """The norm factor against torch's RMSNorm (no gain) in fp64, closed forms
    for constant and zero rows, and exact homogeneity at eps = 0."""
    rng = np.random.default_rng(30)
    Z = rng.standard_normal((5, 96))
    eps = 1e-6
    f = orc.inv_rms_rows(Z, eps)
    want = torch.nn.functional.rms_norm(torch.from_numpy(Z), (96,), eps=eps).numpy()
    assert np.allclose(Z * f[:, None], want, rtol=1e-14, atol=1e-15)
    assert math.isclose(orc.inv_rms_rows(np.full((1, 64), 3.0), 0.5)[0], 1 / math.sqrt(9.5), rel_tol=1e-15)
    assert np.allclose(orc.inv_rms_rows(4.0 * Z, 0.0), orc.inv_rms_rows(Z, 0.0) / 4.0, rtol=1e-15, atol=0)
    assert orc.inv_rms_rows(np.zeros((1, 64)), 1e-6)[0] == 1 / math.sqrt(1e-6)


def test_rope_definition(orc):
    """Rotary positions: identity at position 0; pair i of each head equals the
    complex product (v[2i] + i v[2i+1]) e^(i theta); closed-form angles
    (pair 0 turns by pos radians; hd = 4, base 100: pair 1 by pos / 10);
    q . k depends on the two positions only through their difference."""
    rng = np.random.default_rng(31)
    nh, hd = 3, 16
    V = rng.standard_normal((4, nh * hd))
    pos = np.array([0, 1, 37, 2661], np.int32)
    R = orc.rope_rows(V, nh, hd, pos, 10000.0)
    assert np.array_equal(R[0], V[0])
    for r in range(4):
        z = V[r].reshape(nh, hd // 2, 2) @ np.array([1, 1j])
        w = z * np.exp(1j * pos[r] * 10000.0 ** (-np.arange(hd // 2) * 2.0 / hd))
        got = R[r].reshape(nh, hd // 2, 2)
        assert np.allclose(got[..., 0], w.real, rtol=0, atol=1e-12)
        assert np.allclose(got[..., 1], w.imag, rtol=0, atol=1e-12)
    e = orc.rope_rows(np.array([[1.0, 0.0, 1.0, 0.0]]), 1, 4, [10], 100.0)[0]
    assert np.allclose(e, [math.cos(10), math.sin(10), math.cos(1), math.sin(1)], rtol=0, atol=1e-15)
    q, k = rng.standard_normal((2, hd))

    def dot(pq, pk):
        return orc.rope_rows(q[None], 1, hd, [pq], 500.0)[0] @ orc.rope_rows(k[None], 1, hd, [pk], 500.0)[0]
    for pq, pk, t in [(5, 2, 11), (100, 0, 900), (7, 7, 3)]:
        assert math.isclose(dot(pq, pk), dot(pq + t, pk + t), rel_tol=1e-10, abs_tol=1e-12)


# ----------------------------------------------------------------------------- decode step
def _small_layer(orc, rng, w_dtype=1, kv_dtype=1, act_fp8=0, D=128, nq=4, nkv=2, d=64, F=256,
                 lens=(1, 5, 33, 64, 70)):
    gen = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    act = 0 if w_dtype == 0 else 1

    def W(r, c):
        v = torch.randn((r, c), generator=gen) * 0.02
        s = wl.fp8_scale(v) if w_dtype == 2 else 1.0
        return wl.to_numpy_codes(wl.encode(v, w_dtype, s), w_dtype), s
    wq, sq = W((nq + 2 * nkv) * d, D)
    wo, so = W(D, nq * d)
    wg, sg = W(2 * F, D)
    wd, sd = W(D, F)
    hist_vals_k = [torch.randn((L - 1, nkv, d), generator=gen) for L in lens]
    hist_vals_v = [torch.randn((L - 1, nkv, d), generator=gen) for L in lens]
    ks = wl.fp8_scale(torch.cat(hist_vals_k)) if kv_dtype == 2 else 1.0
    vs = wl.fp8_scale(torch.cat(hist_vals_v)) if kv_dtype == 2 else 1.0
    hk = [wl.to_numpy_codes(wl.encode(t, kv_dtype, ks), kv_dtype) for t in hist_vals_k]
    hv = [wl.to_numpy_codes(wl.encode(t, kv_dtype, vs), kv_dtype) for t in hist_vals_v]
    layer = dict(hidden=D, n_q=nq, n_kv=nkv, head_dim=d, ffn=F, w_dtype=w_dtype, w_qkv=wq, w_o=wo,
                 w_gu=wg, w_d=wd, s_qkv=sq, s_o=so, s_gu=sg, s_d=sd, act_dtype=act,
                 act_fp8=act_fp8, kv_dtype=kv_dtype, k_scale=ks, v_scale=vs)
    x = torch.randn((len(lens), D), generator=gen).numpy()
    hist = orc.History(hk, hv, kv_dtype, nkv, d)
    return layer, hist, np.arange(len(lens)), np.asarray(lens) - 1, x


def test_step_zero_gate_gives_h(orc):
    rng = np.random.default_rng(20)
    layer, hist, seq, pos, x = _small_layer(orc, rng)
    layer["w_gu"] = np.zeros_like(layer["w_gu"])
    out = orc.decode_step(layer, hist, seq, pos, x)
    assert not out["a"].any()
    assert np.array_equal(out["y"], out["h"])


def test_step_zero_wo_gives_x(orc):
    rng = np.random.default_rng(21)
    layer, hist, seq, pos, x = _small_layer(orc, rng)
    layer["w_o"] = np.zeros_like(layer["w_o"])
    out = orc.decode_step(layer, hist, seq, pos, x)
    assert np.array_equal(out["h"], x.astype(np.float64))


def test_step_zero_query_gives_mean_value(orc):
    """q rows of W_qkv set to zero: every head's attention is the plain mean of
    its kv head's values over positions 0..p, including the appended value."""
    rng = np.random.default_rng(22)
    layer, hist, seq, pos, x = _small_layer(orc, rng, w_dtype=0, kv_dtype=0)
    nq, nkv, d = layer["n_q"], layer["n_kv"], layer["head_dim"]
    layer["w_qkv"] = layer["w_qkv"].copy()
    layer["w_qkv"][:nq * d] = 0
    out = orc.decode_step(layer, hist, seq, pos, x)
    for r in range(len(seq)):
        vnew = out["qkv"][r, (nq + nkv) * d:].reshape(nkv, d)
        Vh = hist.v[hist.hist_off[r]:hist.hist_off[r] + hist.hist_len[r]].astype(np.float64)
        allv = np.concatenate([Vh, vnew[None]], 0)
        for h in range(nq):
            want = allv[:, h // (nq // nkv)].mean(0)
            got = out["attn"][r].reshape(nq, d)[h]
            assert np.allclose(got, want.astype(np.float32), rtol=1e-6, atol=1e-7)


def test_step_vs_torch_composition(orc):
    """bf16 tier against a composition of torch CPU library ops in fp64 (matmul,
    scaled_dot_product_attention, silu) with bf16 rounding at the same points."""
    rng = np.random.default_rng(23)
    layer, hist, seq, pos, x = _small_layer(orc, rng)
    D, nq, nkv, d, F = (layer[k] for k in ("hidden", "n_q", "n_kv", "head_dim", "ffn"))
    out = orc.decode_step(layer, hist, seq, pos, x)

    def bf(t):
        return t.to(torch.bfloat16).double()

    def Wt(name):
        return torch.from_numpy(layer[name].view(np.int16).copy()).view(torch.bfloat16).double()
    X = torch.from_numpy(x).double()
    qkv = bf(bf(X) @ Wt("w_qkv").T)
    assert np.allclose(out["qkv"], qkv.numpy(), rtol=2 ** -7, atol=1e-6)
    qkv = torch.from_numpy(out["qkv"])  # continue from the oracle's stored values
    att = []
    for r in range(len(seq)):
        o, L = hist.hist_off[r], hist.hist_len[r]
        Kh = torch.from_numpy(hist.k[o:o + L].view(np.int16).copy()).view(torch.bfloat16).double()
        Vh = torch.from_numpy(hist.v[o:o + L].view(np.int16).copy()).view(torch.bfloat16).double()
        kn = qkv[r, nq * d:(nq + nkv) * d].reshape(1, nkv, d)
        vn = qkv[r, (nq + nkv) * d:].reshape(1, nkv, d)
        K = torch.cat([Kh, kn]).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
        V = torch.cat([Vh, vn]).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
        qh = qkv[r, :nq * d].reshape(nq, 1, d)
        att.append(torch.nn.functional.scaled_dot_product_attention(qh, K, V)[:, 0].reshape(-1))
    att = bf(torch.stack(att))
    assert np.allclose(out["attn"], att.numpy(), rtol=2 ** -7, atol=1e-6)
    att = torch.from_numpy(out["attn"])
    h = X + att @ Wt("w_o").T
    assert np.allclose(out["h"], h.numpy(), rtol=1e-10, atol=1e-12)
    gu = bf(h) @ Wt("w_gu").T
    a = bf(torch.nn.functional.silu(gu[:, :F]) * gu[:, F:])
    assert np.allclose(out["a"], a.numpy(), rtol=2 ** -7, atol=1e-7)
    y = h + torch.from_numpy(out["a"]) @ Wt("w_d").T
    assert np.allclose(out["y"], y.numpy(), rtol=1e-10, atol=1e-12)


def _fold_gains(layer, rng):
    """Turns on the norm and rotary positions and folds random norm gains into
    the f32 W_qkv and W_gate_up columns; returns the two gain vectors."""
    D = layer["hidden"]
    g1 = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    g2 = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    layer["w_qkv"] = (layer["w_qkv"].astype(np.float32) * g1[None, :]).astype(np.float32)
    layer["w_gu"] = (layer["w_gu"].astype(np.float32) * g2[None, :]).astype(np.float32)
    layer.update(norm=True, rope=True, norm_eps=1e-6, rope_base=10000.0)
    return g1, g2


def test_step_norm_rope_vs_torch_composition(orc):
    """f32 tier with RMSNorm and rotary positions, against torch fp64: rms_norm
    with the gain and the unfolded weights, the rotation as a complex product,
    scaled_dot_product_attention, silu; f32 rounding at the same points."""
    rng = np.random.default_rng(26)
    layer, hist, seq, pos, x = _small_layer(orc, rng, w_dtype=0, kv_dtype=0)
    W0 = {k: layer[k].astype(np.float64) for k in ("w_qkv", "w_o", "w_gu", "w_d")}
    g1, g2 = _fold_gains(layer, rng)
    D, nq, nkv, d, F = (layer[k] for k in ("hidden", "n_q", "n_kv", "head_dim", "ffn"))
    out = orc.decode_step(layer, hist, seq, pos, x)

    def f32(t):
        return t.float().double()
    X = torch.from_numpy(x).double()
    xn = torch.nn.functional.rms_norm(X, (D,), weight=torch.from_numpy(g1).double(), eps=1e-6)
    qkv = (xn @ torch.from_numpy(W0["w_qkv"]).T).numpy()
    for r in range(len(seq)):
        z = qkv[r, :(nq + nkv) * d].reshape(nq + nkv, d // 2, 2) @ np.array([1, 1j])
        z = z * np.exp(1j * pos[r] * 10000.0 ** (-np.arange(d // 2) * 2.0 / d))
        qkv[r, :(nq + nkv) * d] = np.stack([z.real, z.imag], -1).reshape(-1)
    qkv = f32(torch.from_numpy(qkv))
    assert np.allclose(out["qkv"], qkv.numpy(), rtol=1e-6, atol=1e-7)
    qkv = torch.from_numpy(out["qkv"])
    att = []
    for r in range(len(seq)):
        o, L = hist.hist_off[r], hist.hist_len[r]
        Kh = torch.from_numpy(hist.k[o:o + L].astype(np.float64))
        Vh = torch.from_numpy(hist.v[o:o + L].astype(np.float64))
        kn = qkv[r, nq * d:(nq + nkv) * d].reshape(1, nkv, d)
        vn = qkv[r, (nq + nkv) * d:].reshape(1, nkv, d)
        K = torch.cat([Kh, kn]).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
        V = torch.cat([Vh, vn]).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
        qh = qkv[r, :nq * d].reshape(nq, 1, d)
        att.append(torch.nn.functional.scaled_dot_product_attention(qh, K, V)[:, 0].reshape(-1))
    att = f32(torch.stack(att))
    assert np.allclose(out["attn"], att.numpy(), rtol=1e-6, atol=1e-7)
    h = X + torch.from_numpy(out["attn"]) @ torch.from_numpy(W0["w_o"]).T
    assert np.allclose(out["h"], h.numpy(), rtol=1e-10, atol=1e-12)
    hn = torch.nn.functional.rms_norm(f32(h), (D,), weight=torch.from_numpy(g2).double(), eps=1e-6)
    gu = hn @ torch.from_numpy(W0["w_gu"]).T
    a = f32(torch.nn.functional.silu(gu[:, :F]) * gu[:, F:])
    assert np.allclose(out["a"], a.numpy(), rtol=1e-6, atol=1e-7)


def test_step_fp8_tier_projection(orc):
    """fp8 matrix-core tier: a projection is s_z * s_W * sum(z8 * W8) with the
    input quantised per row; checked on W_qkv against numpy on decoded codes."""
    rng = np.random.default_rng(24)
    layer, hist, seq, pos, x = _small_layer(orc, rng, w_dtype=2, kv_dtype=2, act_fp8=1)
    out = orc.decode_step(layer, hist, seq, pos, x)
    Wv = orc.e4m3_value(layer["w_qkv"])
    for r in range(len(seq)):
        codes, s = orc.act_quant(x[r].astype(np.float64))
        want = (orc.e4m3_value(codes) @ Wv.T) * layer["s_qkv"] * s
        got = out["qkv"][r]
        assert np.allclose(got, want, rtol=2 ** -7, atol=1e-6)


def test_step_fp8_tier_composition(orc):
    """fp8 tier, every stage, against torch fp64 library ops on decoded codes.
    Each projection input is quantised per row: s = fp32(max|z|) / 448 (fp32
    division), codes = torch's E4M3 conversion of z / s (fp32 division,
    clamped to +-448 first), and the projection is s * s_W * (codes @ W8^T).
    The quantised z is the f32 residual-stream value for x and h, and the
    stored bf16 value for attn and a.  The row's key and value are appended
    as E4M3 of (stored bf16 value) / scale in fp32; attention is torch's SDPA
    over decoded K, V times their scales.  Stored outputs (qkv, attn, a) are
    bf16; h and y stay in fp64.  Each stage starts from the oracle's stored
    values of the previous one, so a rounding flip cannot cascade."""
    rng = np.random.default_rng(27)
    layer, hist, seq, pos, x = _small_layer(orc, rng, w_dtype=2, kv_dtype=2, act_fp8=1)
    D, nq, nkv, d, F = (layer[k] for k in ("hidden", "n_q", "n_kv", "head_dim", "ffn"))
    out = orc.decode_step(layer, hist, seq, pos, x)
    e4 = torch.float8_e4m3fn

    def bf(t):
        return t.to(torch.bfloat16).double()

    def W8(name, sname):
        return torch.from_numpy(layer[name].copy()).view(e4).double() * float(layer[sname])

    def proj(z32, name, sname):
        z32 = z32.float()
        s = z32.abs().amax(1, keepdim=True) / torch.tensor(448.0, dtype=torch.float32)
        s = torch.where(s > 0, s, torch.ones_like(s))
        codes = (z32 / s).clamp(-448.0, 448.0).to(e4).double()
        return s.double() * (codes @ W8(name, sname).T)

    def stored_bf16(a):  # oracle's stored bf16 values are exact in f32
        return torch.from_numpy(a).float()
    X = torch.from_numpy(x).float()
    qkv = bf(proj(X, "w_qkv", "s_qkv"))
    assert np.allclose(out["qkv"], qkv.numpy(), rtol=2 ** -7, atol=1e-6)
    qkv = torch.from_numpy(out["qkv"])
    ks, vs = float(layer["k_scale"]), float(layer["v_scale"])

    def append(vals, sc):  # E4M3 of value / scale in fp32, decoded times the scale
        return (vals.float() / torch.tensor(sc, dtype=torch.float32)).clamp(-448.0, 448.0).to(e4).double() * sc
    att = []
    for r in range(len(seq)):
        o, L = hist.hist_off[r], hist.hist_len[r]
        Kh = torch.from_numpy(hist.k[o:o + L].copy()).view(e4).double() * ks
        Vh = torch.from_numpy(hist.v[o:o + L].copy()).view(e4).double() * vs
        kn = append(qkv[r, nq * d:(nq + nkv) * d].reshape(1, nkv, d), ks)
        vn = append(qkv[r, (nq + nkv) * d:].reshape(1, nkv, d), vs)
        K = torch.cat([Kh, kn]).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
        V = torch.cat([Vh, vn]).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
        qh = qkv[r, :nq * d].reshape(nq, 1, d)
        att.append(torch.nn.functional.scaled_dot_product_attention(qh, K, V)[:, 0].reshape(-1))
    att = bf(torch.stack(att))
    assert np.allclose(out["attn"], att.numpy(), rtol=2 ** -7, atol=1e-6)
    h = X.double() + proj(stored_bf16(out["attn"]), "w_o", "s_o")
    assert np.allclose(out["h"], h.numpy(), rtol=1e-10, atol=1e-12)
    gu = proj(torch.from_numpy(out["h"]).float(), "w_gu", "s_gu")
    a = bf(torch.nn.functional.silu(gu[:, :F]) * gu[:, F:])
    assert np.allclose(out["a"], a.numpy(), rtol=2 ** -7, atol=1e-7)
    y = torch.from_numpy(out["h"]) + proj(stored_bf16(out["a"]), "w_d", "s_d")
    assert np.allclose(out["y"], y.numpy(), rtol=1e-10, atol=1e-12)
    # the per-row scale matters: one scale over the whole batch gives other h
    z = stored_bf16(out["attn"])
    s_all = z.abs().amax() / torch.tensor(448.0, dtype=torch.float32)
    h_tensor = X.double() + s_all.double() * ((z / s_all).clamp(-448, 448).to(e4).double() @ W8("w_o", "s_o").T)
    assert not np.allclose(out["h"], h_tensor.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("norm_rope", [False, True])
def test_step_rows_independent_and_sequential(orc, norm_rope):
    """Rows are independent (any order, alone) and several rows of one sequence
    in one step equal the same rows run one step at a time (with rotary
    positions too: the stored keys are the rotated ones)."""
    rng = np.random.default_rng(25)
    layer, hist, seq, pos, x = _small_layer(orc, rng)
    if norm_rope:
        layer.update(norm=True, rope=True, norm_eps=1e-6, rope_base=10000.0)
    full = orc.decode_step(layer, hist, seq, pos, x)
    perm = np.asarray([4, 2, 0, 3, 1])
    sh = orc.decode_step(layer, hist, seq[perm], pos[perm], x[perm])
    assert np.array_equal(sh["y"], full["y"][perm])
    alone = orc.decode_step(layer, hist, seq[3:4], pos[3:4], x[3:4])
    assert np.array_equal(alone["y"][0], full["y"][3])
    # four rows of sequence 2 (positions 32..35) in one step ...
    nq, nkv, d = layer["n_q"], layer["n_kv"], layer["head_dim"]
    base = 32
    s2k = hist.k[hist.hist_off[2]:hist.hist_off[2] + base]
    s2v = hist.v[hist.hist_off[2]:hist.hist_off[2] + base]
    h1 = orc.History([s2k], [s2v], 1, nkv, d)
    xs = rng.standard_normal((4, layer["hidden"])).astype(np.float32)
    one = orc.decode_step(layer, h1, [0] * 4, base + np.arange(4), xs)
    # ... equal four one-row steps, each on the history grown by the previous rows
    kk = orc.bf16_round(one["qkv"][:, nq * d:(nq + nkv) * d]).reshape(4, nkv, d)
    vv = orc.bf16_round(one["qkv"][:, (nq + nkv) * d:]).reshape(4, nkv, d)
    for j in range(4):
        hj = orc.History([np.concatenate([s2k, kk[:j]])], [np.concatenate([s2v, vv[:j]])], 1, nkv, d)
        r = orc.decode_step(layer, hj, [0], [base + j], xs[j:j + 1])
        assert np.array_equal(r["y"][0], one["y"][j])


# ----------------------------------------------------------------------------- brute force in long double
def _brute_step(layer, hist, seq, pos, x):
    """The whole step written out with numpy long-double loops, f32 tier: the
    stored weights, qkv rounded to f32 (after the norm factor and rotary
    positions when on), every row appended before any row attends, softmax
    with the maximum subtracted, attn and a rounded to f32, f32 residual
    inputs.  Independent of the C oracle's code."""
    LD = np.longdouble
    D, nq, nkv, d, F = (layer[k] for k in ("hidden", "n_q", "n_kv", "head_dim", "ffn"))
    f32 = lambda v: np.asarray(v, np.float32).astype(LD)
    Wq, Wo, Wg, Wd = (layer[k].astype(LD) for k in ("w_qkv", "w_o", "w_gu", "w_d"))
    n = len(seq)
    X = x.astype(LD)

    def inv_rms(z):
        return LD(1) / np.sqrt(np.sum(z * z) / LD(len(z)) + LD(layer.get("norm_eps", 1e-6)))

    def rope(v, p):
        out = v.copy()
        base = LD(layer.get("rope_base", 10000.0))
        for i in range(d // 2):
            th = LD(p) * base ** (LD(-2 * i) / LD(d))
            c, s = np.cos(th), np.sin(th)
            for h in range(nq + nkv):
                a, b = v[h * d + 2 * i], v[h * d + 2 * i + 1]
                out[h * d + 2 * i], out[h * d + 2 * i + 1] = a * c - b * s, a * s + b * c
        return out
    qkv = []
    for r in range(n):
        v = Wq @ f32(x[r])
        if layer.get("norm"):
            v = v * inv_rms(X[r])
        if layer.get("rope"):
            v = rope(v, pos[r])
        qkv.append(f32(v))
    qkv = np.stack(qkv)
    K = {s: [hist.k[hist.hist_off[s] + t].astype(LD) for t in range(hist.hist_len[s])] for s in set(seq)}
    V = {s: [hist.v[hist.hist_off[s] + t].astype(LD) for t in range(hist.hist_len[s])] for s in set(seq)}
    for r in range(n):
        s, p = seq[r], pos[r]
        kr = qkv[r, nq * d:(nq + nkv) * d].reshape(nkv, d)
        vr = qkv[r, (nq + nkv) * d:].reshape(nkv, d)
        while len(K[s]) <= p:
            K[s].append(None)
            V[s].append(None)
        K[s][p], V[s][p] = kr, vr
    G = nq // nkv
    attn = np.zeros((n, nq * d), LD)
    for r in range(n):
        s, p = seq[r], pos[r]
        for h in range(nq):
            g = h // G
            q = qkv[r, h * d:(h + 1) * d]
            sc = np.array([np.sum(q * K[s][t][g]) / np.sqrt(LD(d)) for t in range(p + 1)], LD)
            w = np.exp(sc - sc.max())
            w = w / w.sum()
            attn[r, h * d:(h + 1) * d] = sum(w[t] * V[s][t][g] for t in range(p + 1))
    attn = f32(attn)
    h = X + attn @ Wo.T
    hin = f32(h)
    gu = hin @ Wg.T
    if layer.get("norm"):
        fac = np.array([inv_rms(h[r]) for r in range(n)], LD)
        gu = gu * fac[:, None]
    a = f32(gu[:, :F] / (LD(1) + np.exp(-gu[:, :F])) * gu[:, F:])
    y = h + a @ Wd.T
    return dict(qkv=qkv, attn=attn, h=h, a=a, y=y)


@pytest.mark.parametrize("norm_rope", [False, True])
def test_step_vs_long_double_brute_force(orc, norm_rope):
    """The C oracle's whole step against a numpy long-double brute force on a
    tiny f32 layer (several rows of one sequence, GQA): the f32-rounded
    intermediates equal, h and y within 1e-12 relative."""
    rng = np.random.default_rng(40)
    layer, hist, seq, pos, x = _small_layer(orc, rng, w_dtype=0, kv_dtype=0, D=64, nq=4, nkv=2, d=16, F=64,
                                            lens=(1, 5, 33))
    if norm_rope:
        layer.update(norm=True, rope=True, norm_eps=1e-6, rope_base=10000.0)
    seq = np.asarray([0, 1, 2, 2], np.int32)
    pos = np.asarray([0, 4, 32, 33], np.int32)
    x = np.concatenate([x, x[2:3] * 0.5], 0).astype(np.float32) * 2.0
    out = orc.decode_step(layer, hist, seq, pos, x)
    want = _brute_step(layer, hist, seq, pos, x)
    for k in ("qkv", "attn", "a"):
        assert np.array_equal(out[k], want[k].astype(np.float64)), k
    for k in ("h", "y"):
        ref = want[k].astype(np.float64)
        assert np.allclose(out[k], ref, rtol=1e-12, atol=1e-13), k
