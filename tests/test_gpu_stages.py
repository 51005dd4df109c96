"""Stage parity of the decode step against the fp64 oracle, on every workload.

Each stage of the step runs on the GPU at full batch, in the launch
configuration the benchmark times (same rows, same engine: K splits fixed for
the workload's batch, fused append for pure decode batches), with the sampled
rows carrying the oracle's stored values of the previous stage.  Every stage
is then compared with the oracle's value of that stage on those rows:

  - before rounding: the stage with an f32 output against the oracle's exact
    value of the stage (max |g - e| / max |e| per row, gate per stage below);
  - stored (bf16): every element equals the oracle's stored value, or is the
    adjacent bf16 value while the exact value lies within the stage's gate of
    the midpoint between the two (a rounding decision that the accumulation
    error may legitimately flip), and never anything else;
  - h and y (f32 residual stream): max |g - e| / max |e| per row within the
    gate.

The chained step (each stage fed the GPU's own previous stage) is reported
and held only to a sanity bound: the oracle's own output moves by about the
spec bar under a 1e-6 relative perturbation of x (a single flipped bf16
or fp8 decision propagates through every later projection), so the chained
comparison cannot resolve errors below the bar.

Gates (per-row max error over max magnitude, before rounding):
  - projections with exact products and fp32 accumulation (vector GEMV,
    matrix-core bf16, fp8 decoded to bf16): 2e-5.  K = 3,584 to 18,944 fp32
    additions of products give a typical relative error of sqrt(K) x 2^-24,
    1e-6 to 8e-6 of the sum's own scale;
  - native fp8 matrix-core instruction: 2e-4 (each instruction sums its 128
    products with about 17 significant bits, ~2e-5 of a projection);
  - attention: 1e-4 (fp32 online softmax; the probabilities enter the P.V
    product as a hi + lo bf16 pair, about 16 significant bits).
The spec bars (2e-3 bf16, 3e-2 fp8) are far above every gate.
"""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

BAR = {wl.F32: 2e-3, wl.BF16: 2e-3, wl.FP8: 3e-2}
GATE_PROJ = {0: 2e-5, 1: 2e-5, 2: 2e-4, 3: 2e-5}
GATE_ATTN = 1e-4
GATE_F32_TIER = 1e-5
CHAIN_SANITY = 10.0  # chained-step bound, in units of the bar


@pytest.fixture(scope="module")
def H():
    import gpu_harness
    return gpu_harness


def row_err(got, want):
    got = np.asarray(got, np.float64).reshape(len(got), -1)
    want = np.asarray(want, np.float64).reshape(len(want), -1)
    den = np.abs(want).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return np.abs(got - want).max(axis=1) / den


def check_stored_bf16(orc, got, want, exact, gate, label):
    """got, want: stored bf16 values [rows][m]; exact: the oracle's value of
    the stage before rounding.  Every stored value must be the bf16 rounding
    (RNE) of some number within `gate` x max|exact| (per row) of the exact
    value, i.e. lie between the roundings of exact - tol and exact + tol; it
    differs from the oracle's stored value only where such a number rounds the
    other way (a rounding decision the accumulation error may flip)."""
    got = np.asarray(got, np.float64).reshape(len(got), -1)
    want = np.asarray(want, np.float64).reshape(len(want), -1)
    exact = np.asarray(exact, np.float64).reshape(len(exact), -1)
    assert np.isfinite(got).all(), label
    tol = gate * np.abs(exact).max(axis=1, keepdims=True)
    lo = orc.bf16_value(orc.bf16_round(exact - tol))
    hi = orc.bf16_value(orc.bf16_round(exact + tol))
    bad = (got < lo) | (got > hi)
    assert not bad.any(), f"{label}: {int(bad.sum())} stored values are not a rounding of a value within the gate"
    flips = int((got != want).sum())
    frac = flips / max(got.size, 1)
    print(f"  {label}: {flips} of {got.size} stored values differ from the oracle's (rounding flips, {frac:.2e})",
          flush=True)
    return frac


def oracle_rows(orc, w, rows):
    rows = np.asarray(rows)
    seqs = np.unique(w.seq[rows])
    hk, hv = wl.history_lists(w, seqs)
    hist = orc.History(hk, hv, w.kv_dtype, w.n_kv, w.head_dim)
    x = w.x[torch.as_tensor(rows)].cpu().numpy()
    return orc.decode_step(wl.layer_dict(w), hist, w.seq[rows], w.pos[rows], x, raw=True)


def sample_rows(w, k, seed, chunk_rows=0):
    """k random rows that are not rows of the prompt slice, plus the first
    `chunk_rows` rows of the slice (the oracle needs every earlier slice row)."""
    rng = np.random.default_rng(seed)
    slice_seq = w.seq.max() if chunk_rows else None
    decode = np.nonzero(w.seq != slice_seq)[0] if chunk_rows else np.arange(w.n_rows)
    pick = set(rng.choice(decode, size=min(k, len(decode)), replace=False).tolist())
    if chunk_rows:
        pick |= set(np.nonzero(w.seq == slice_seq)[0][:chunk_rows].tolist())
    return sorted(pick)


def run_stages(H, orc, w, layer, rows, label):
    """The stage chain at full batch with the sampled rows fed the oracle's
    values; returns the per-stage errors of the sampled rows."""
    import paged_kv_decode_attn_amd as pkd
    L = layer.layer
    fam = int(L.w_qkv.family)
    n, D, nq, nkv, d, F = w.n_rows, w.hidden, w.n_q, w.n_kv, w.head_dim, w.ffn
    nqkv = (nq + 2 * nkv) * d
    act = w.act_dtype
    fp8 = w.w_dtype == wl.FP8
    f32_tier = act == wl.F32
    R = torch.as_tensor(np.asarray(rows), device="cuda")
    o = oracle_rows(orc, w, rows)
    gate_p = GATE_F32_TIER if f32_tier else GATE_PROJ[fam]
    res = {}

    def stored_codes(vals):  # oracle stored values -> device tensor of act-dtype codes
        if act == wl.F32:
            return torch.from_numpy(np.asarray(vals, np.float32)).cuda()
        return torch.from_numpy(orc.bf16_round(vals).view(np.int16).copy()).cuda()

    def put(t, vals):
        t = t.clone()
        t[R] = stored_codes(vals).reshape(t[R].shape)
        return t

    wsb = max(pkd.pkd_gemv_workspace_bytes(M, n) for M in (L.w_qkv, L.w_o, L.w_gate_up, L.w_down))
    ws = H.aligned_empty(wsb) if wsb else None

    def proj(M, xin, xdt, nout, out_dtype, residual=None, silu=False, y_bf16=None, **ep):
        tdt = torch.float32 if out_dtype == wl.F32 else torch.int16
        y = torch.empty((n, nout), dtype=tdt, device="cuda")
        pkd.gemv_rows(M, xin, xdt, n, y, out_dtype, residual, silu, y_bf16, ws=ws, **ep)
        return y

    def stored_stage(name, M, xin, xdt, nout, exact, stored, gate, **kw):
        """Runs a stored-output projection twice (f32, then the stored dtype)."""
        y32 = proj(M, xin, xdt, nout, wl.F32, **kw)
        ya = proj(M, xin, xdt, nout, act, **kw) if act != wl.F32 else y32
        torch.cuda.synchronize()
        g32 = H.values(y32[R], wl.F32)
        res[name + "_f32"] = float(row_err(g32, exact).max())
        print(f"  {label} {name} before rounding: {res[name + '_f32']:.2e} (gate {gate:.0e})", flush=True)
        assert res[name + "_f32"] <= gate, (label, name, res[name + "_f32"])
        if act != wl.F32:
            res[name + "_flips"] = check_stored_bf16(orc, H.values(ya[R], wl.BF16), stored, exact, gate,
                                                     f"{label} {name}")
        return ya

    x = w.x.cuda().contiguous()
    # With norms and rotary positions the projections take the library's own
    # per-row 1/rms factors and rotary table, as the step does; the oracle's
    # stage values include both.
    def inv_rms(z):
        f = torch.empty(n, dtype=torch.float32, device="cuda")
        pkd.rms_norm_factor(z, n, D, w.norm_eps, f)
        return f
    ep_qkv, ep_gu = {}, {}
    if w.norm:
        ep_qkv["row_scale"] = inv_rms(x)
    if w.rope:
        cs = torch.empty((n, d // 2, 2), dtype=torch.float32, device="cuda")
        pkd.rope_table(torch.as_tensor(np.asarray(w.pos, np.int32), device="cuda"), n, d, w.rope_base, cs)
        ep_qkv.update(rope_cs=cs, rope_cols=(nq + nkv) * d, rope_head_dim=d)
    # ---- qkv = W_qkv x (the bf16 tier takes x rounded to bf16; fp8 quantises f32 x per row)
    if fp8 or f32_tier:
        xin, xdt = x, wl.F32
    else:
        xin, xdt = x.to(torch.bfloat16).view(torch.int16).contiguous(), wl.BF16
    qkv = stored_stage("qkv", L.w_qkv, xin, xdt, nqkv, o["qkv_raw"], o["qkv"], gate_p, **ep_qkv)
    # ---- append + attention, the sampled rows' q, k, v from the oracle
    qkv_in = put(qkv, o["qkv"]).view(n, nq + 2 * nkv, d)
    q, k, v = (qkv_in[:, :nq].contiguous(), qkv_in[:, nq:nq + nkv].contiguous(),
               qkv_in[:, nq + nkv:].contiguous())
    pool = H.GpuPool(w)
    distinct = len(set(w.seq.tolist())) == n
    gate_a = GATE_F32_TIER if f32_tier else GATE_ATTN
    a32 = H.run_attention(pool, w.seq, w.pos, q, k, v, wl.F32, distinct).view(n, nq * d)
    res["attn_f32"] = float(row_err(H.values(a32[R], wl.F32), o["attn_raw"]).max())
    print(f"  {label} attn before rounding: {res['attn_f32']:.2e} (gate {gate_a:.0e})", flush=True)
    assert res["attn_f32"] <= gate_a, (label, "attn", res["attn_f32"])
    if act != wl.F32:
        # again with the stored output (the appends write the same bytes again)
        att = H.run_attention(pool, w.seq, w.pos, q, k, v, act, distinct).view(n, nq * d)
        res["attn_flips"] = check_stored_bf16(orc, H.values(att[R], wl.BF16), o["attn"], o["attn_raw"], gate_a,
                                              f"{label} attn")
    else:
        att = a32
    pkd.pkd_pool_check(pool.handle)
    del pool
    # ---- h = x + W_o attn
    hb = torch.empty((n, D), dtype=torch.int16, device="cuda")
    h = proj(L.w_o, put(att, o["attn"]), act, D, wl.F32, residual=x,
             y_bf16=None if (fp8 or f32_tier) else hb)
    torch.cuda.synchronize()
    res["h"] = float(row_err(H.values(h[R], wl.F32), o["h"]).max())
    print(f"  {label} h: {res['h']:.2e} (gate {gate_p:.0e})", flush=True)
    assert res["h"] <= gate_p, (label, "h", res["h"])
    # the bf16 copy of h that the next projection takes is the RNE of the f32 h
    if not (fp8 or f32_tier):
        assert torch.equal(hb, h.to(torch.bfloat16).view(torch.int16)), label
    if F:
        hf = h.clone()
        hf[R] = torch.from_numpy(o["h"].astype(np.float32)).cuda()
        if fp8 or f32_tier:
            hin, hdt = hf, wl.F32
        else:
            hin, hdt = put(hb, o["h"]), wl.BF16
        if w.norm:
            ep_gu["row_scale"] = inv_rms(hf)
        # ---- a = silu(W_g h) * (W_u h)
        a = stored_stage("a", L.w_gate_up, hin, hdt, F, o["a_raw"], o["a"], gate_p, silu=True, **ep_gu)
        # ---- y = h + W_d a
        y = proj(L.w_down, put(a, o["a"]), act, D, wl.F32, residual=hf)
        torch.cuda.synchronize()
        res["y"] = float(row_err(H.values(y[R], wl.F32), o["y"]).max())
        print(f"  {label} y: {res['y']:.2e} (gate {gate_p:.0e})", flush=True)
        assert res["y"] <= gate_p, (label, "y", res["y"])
    print(f"{label} stage errors: " + ", ".join(f"{k} {v:.2e}" for k, v in res.items()), flush=True)
    return o, res


def chained(H, w, layer, pool, rows, o, label):
    y = layer.step(pool, w.seq, w.pos, w.x).cpu().numpy()
    assert np.isfinite(y).all()
    e = float(row_err(y[rows], o["y"]).max())
    bar = BAR[w.w_dtype]
    print(f"{label} chained step y: max rel err {e:.3e} (bar {bar:.0e}; reported, sanity bound "
          f"{CHAIN_SANITY:.0f}x)", flush=True)
    assert e <= CHAIN_SANITY * bar, label
    return e


def full_case(H, orc, name, kw, rows_fn, device="cpu", norm_rope=False):
    w = wl.make(name, device, **kw)
    if norm_rope:
        w = wl.with_norm_rope(w)
    label = f"{w.name} ({w.n_rows} rows, family {w.family})"
    print(f"workload {label}", flush=True)
    hint = w.n_rows if w.family in (wl.MFMA, wl.MFMA_FP8) else None
    layer = H.GpuLayer(w, batch_hint=hint)
    rows = rows_fn(w)
    o, res = run_stages(H, orc, w, layer, rows, label)
    chained(H, w, layer, H.GpuPool(w), rows, o, label)
    return res


def test_stages_tiny_f32(H, orc):
    full_case(H, orc, "tiny-f32", {}, lambda w: np.arange(w.n_rows))


def test_stages_06b_b1(H, orc):
    full_case(H, orc, "0.6b-b1-bf16", {}, lambda w: [0])


def test_stages_06b_mixed_reduced(H, orc):
    full_case(H, orc, "0.6b-mixed-bf16", dict(n_decode=48, chunk_rows=24, chunk=4, long_max=1400),
              lambda w: np.arange(w.n_rows))


def test_stages_06b_mixed_matrix_core_gemv(H, orc):
    full_case(H, orc, "0.6b-mixed-bf16", dict(n_decode=24, chunk_rows=8, chunk=4, long_max=1400, family=3),
              lambda w: np.arange(w.n_rows))


@pytest.mark.parametrize("family", [1, 2])
def test_stages_fp8_reduced(H, orc, family):
    full_case(H, orc, "7b-b4096-fp8", dict(n=64, L=100, family=family), lambda w: list(range(0, 64, 9)))


@pytest.mark.slow
def test_stages_06b_mixed_full(H, orc):
    full_case(H, orc, "0.6b-mixed-bf16", {}, lambda w: sample_rows(w, 12, 0, chunk_rows=16), device="cuda")


@pytest.mark.slow
def test_stages_7b_b768(H, orc):
    full_case(H, orc, "7b-b768-prefix-bf16", {}, lambda w: sample_rows(w, 10, 1), device="cuda")


@pytest.mark.slow
@pytest.mark.parametrize("family", [1, 2])
def test_stages_7b_fp8_b4096(H, orc, family):
    full_case(H, orc, "7b-b4096-fp8", dict(family=family), lambda w: sample_rows(w, 8, 2), device="cuda")


NORM_ROPE_CASES = [
    ("tiny-f32", {}),
    ("0.6b-mixed-bf16", dict(n_decode=48, chunk_rows=24, chunk=4, long_max=1400)),
    ("0.6b-mixed-bf16", dict(n_decode=48, chunk_rows=24, chunk=4, long_max=1400, family=wl.GEMV)),
    ("7b-b4096-fp8", dict(n=64, L=100)),
    ("7b-b4096-fp8", dict(n=64, L=100, family=wl.MFMA)),
]


@pytest.mark.parametrize("name,kw", NORM_ROPE_CASES)
def test_stages_norm_rope(H, orc, name, kw):
    """With both RMSNorms (1/rms in the projection epilogues, gains folded into
    the weights) and rotary positions on q and k (in the QKV epilogue)."""
    full_case(H, orc, name, kw, lambda w: np.arange(w.n_rows), norm_rope=True)


@pytest.mark.slow
def test_stages_7b_b768_norm_rope(H, orc):
    full_case(H, orc, "7b-b768-prefix-bf16", {}, lambda w: sample_rows(w, 10, 3), device="cuda", norm_rope=True)
