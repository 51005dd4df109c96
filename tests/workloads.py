"""Seeded synthetic inputs shaped like the pages' decode workloads.

This module only draws and places inputs; it holds none of the decode step's
arithmetic.  Both the fp64 oracle and the HIP library are fed from it.
Large normal draws use a seeded torch generator on the requested device;
small integer draws (lengths, page placement) use numpy PCG64.  Stored
formats are produced with torch's own conversions (bf16: round to nearest
even; fp8 E4M3FN: values are scaled into range first, scale = max|v| / 448).

Draw order for a workload with seed s (torch generator seeded s, numpy
PCG64(s)): weights W_qkv, W_o, W_gate_up, W_down (N(0, 0.02^2), row-major),
then lengths and page placement (numpy), then the K history and the V history
(N(0, 1), logical token order), then x (N(0, 1)), then for attention-only
inputs q, k_new, v_new (N(0, 1)).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

F32, BF16, FP8 = 0, 1, 2
GEMV, MFMA, MFMA_FP8 = 0, 1, 2
ESIZE = {F32: 4, BF16: 2, FP8: 1}
TORCH_CODE = {F32: torch.float32, BF16: torch.int16, FP8: torch.uint8}


# --------------------------------------------------------------------------- encoders
def encode(vals: torch.Tensor, dtype: int, scale: float = 1.0) -> torch.Tensor:
    """float32 values -> stored codes (f32 values, bf16 bits as int16, fp8 bits as uint8)."""
    if dtype == F32:
        return vals.float().contiguous()
    if dtype == BF16:
        return vals.to(torch.bfloat16).view(torch.int16).contiguous()
    return (vals / scale).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()


def fp8_scale(vals: torch.Tensor) -> float:
    amax = float(vals.abs().max().item())
    return amax / 448.0 if amax > 0 else 1.0


def to_numpy_codes(t: torch.Tensor, dtype: int) -> np.ndarray:
    a = t.detach().cpu().contiguous().numpy()
    if dtype == BF16:
        return a.view(np.uint16)
    return a


# --------------------------------------------------------------------------- layout
def _k_perm(d: int, dtype: int) -> np.ndarray:
    """Block position of every (token t, dim c) of a K block, [32 * d]."""
    E = 16 // ESIZE[dtype]
    t = np.repeat(np.arange(32), d)
    c = np.tile(np.arange(d), 32)
    vec = ((t // 16) * (d // E) + c // E) * 16 + t % 16
    return vec * E + c % E


def _v_perm(d: int, dtype: int) -> np.ndarray:
    t = np.repeat(np.arange(32), d)
    c = np.tile(np.arange(d), 32)
    a, b, i = t // 16, (t % 16) // 4, t % 4
    if dtype == F32:
        E, vec, el = 4, ((a * (d // 16) + c // 16) * 4 + b) * 16 + c % 16, i
    elif dtype == BF16:
        E, vec, el = 8, ((c // 16) * 4 + b) * 16 + c % 16, 4 * a + i
    else:
        E, vec, el = 16, ((c // 32) * 4 + b) * 16 + c % 16, 8 * ((c // 16) % 2) + 4 * a + i
    return vec * E + el


def fill_pool_pages(pages: torch.Tensor, num_pages: int, n_kv: int, d: int, kv_dtype: int,
                    tables: np.ndarray, counts: np.ndarray, hist_k: torch.Tensor,
                    hist_v: torch.Tensor, hist_off: np.ndarray, hist_len: np.ndarray,
                    poison: bool = True, seqs_per_chunk: int = 256) -> None:
    """Writes every sequence's history into the page region `pages` (a uint8
    tensor of num_pages * n_kv * 2 * block_bytes bytes) following the pool
    layout documented in include/pkd.h.  Unused slots are filled with 0xFF
    bytes (NaN in f32, bf16 and E4M3) when `poison` is set."""
    es = ESIZE[kv_dtype]
    code_t = TORCH_CODE[kv_dtype]
    blk = 32 * d
    view = pages.view(code_t).view(num_pages, n_kv, 2, blk)
    if poison:
        pages.fill_(0xFF)
    dev = pages.device
    kperm = torch.as_tensor(_k_perm(d, kv_dtype), device=dev)
    vperm = torch.as_tensor(_v_perm(d, kv_dtype), device=dev)
    S = len(hist_len)
    for s0 in range(0, S, seqs_per_chunk):
        s1 = min(S, s0 + seqs_per_chunk)
        phys, spans = [], []
        for s in range(s0, s1):
            L = int(hist_len[s])
            npg = (L + 31) // 32
            phys.extend(int(p) for p in tables[s][:npg])
            spans.append((int(hist_off[s]), L, npg))
        if not phys:
            continue
        n = len(phys)
        kk = torch.empty((n, 32, n_kv, d), dtype=code_t, device=dev)
        vv = torch.empty((n, 32, n_kv, d), dtype=code_t, device=dev)
        kk.view(torch.uint8).fill_(0xFF)
        vv.view(torch.uint8).fill_(0xFF)
        j = 0
        for o, L, npg in spans:
            kk[j:j + npg].view(npg * 32, n_kv, d)[:L] = hist_k[o:o + L]
            vv[j:j + npg].view(npg * 32, n_kv, d)[:L] = hist_v[o:o + L]
            j += npg
        # [n][32][n_kv][d] -> [n][n_kv][32*d] in logical (t, c) order, then placed.
        kk = kk.permute(0, 2, 1, 3).reshape(n, n_kv, blk)
        vv = vv.permute(0, 2, 1, 3).reshape(n, n_kv, blk)
        kb = torch.empty_like(kk)
        vb = torch.empty_like(vv)
        kb[:, :, kperm] = kk
        vb[:, :, vperm] = vv
        idx = torch.as_tensor(phys, device=dev, dtype=torch.long)
        view[idx, :, 0] = kb
        view[idx, :, 1] = vb


# --------------------------------------------------------------------------- workloads
@dataclass
class Workload:
    name: str
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    w_dtype: int
    kv_dtype: int
    act_dtype: int
    family: int
    act_fp8: int
    attn_chunk_pages: int
    num_pages: int
    max_seqs: int
    max_pages_per_seq: int
    tables: np.ndarray            # [max_seqs][max_pages_per_seq] int32, -1 unset
    counts: np.ndarray            # [max_seqs] int32
    hist_len: np.ndarray          # [max_seqs] int32
    hist_off: np.ndarray          # [max_seqs] int64
    hist_k: torch.Tensor          # [total][n_kv][d] codes
    hist_v: torch.Tensor
    seq: np.ndarray               # [B] int32
    pos: np.ndarray               # [B] int32
    x: torch.Tensor               # [B][D] f32
    weights: dict = field(default_factory=dict)   # name -> codes tensor [out][in]
    scales: dict = field(default_factory=dict)    # name -> per-tensor scale
    k_scale: float = 1.0
    v_scale: float = 1.0
    q: torch.Tensor | None = None      # attention-only inputs (act-dtype codes)
    k_new: torch.Tensor | None = None
    v_new: torch.Tensor | None = None
    notes: str = ""
    norm: bool = False        # RMSNorm before attention and FFN (gains folded into the weights)
    rope: bool = False        # rotary positions on q and k
    norm_eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def n_rows(self) -> int:
        return int(self.seq.size)

    @property
    def q_dtype(self) -> int:
        return F32 if self.kv_dtype == F32 else BF16


def _weights(gen, dev, w_dtype, shapes) -> tuple[dict, dict]:
    ws, sc = {}, {}
    for name, (rows, cols) in shapes:
        vals = torch.randn((rows, cols), generator=gen, device=dev, dtype=torch.float32) * 0.02
        s = fp8_scale(vals) if w_dtype == FP8 else 1.0
        ws[name] = encode(vals, w_dtype, s)
        sc[name] = s
        del vals
    return ws, sc


def _history(gen, dev, total, n_kv, d, kv_dtype, k_scale=None, v_scale=None):
    hk = torch.randn((max(total, 1), n_kv, d), generator=gen, device=dev, dtype=torch.float32)
    hv = torch.randn((max(total, 1), n_kv, d), generator=gen, device=dev, dtype=torch.float32)
    ks = (k_scale if k_scale is not None else fp8_scale(hk)) if kv_dtype == FP8 else 1.0
    vs = (v_scale if v_scale is not None else fp8_scale(hv)) if kv_dtype == FP8 else 1.0
    return encode(hk, kv_dtype, ks), encode(hv, kv_dtype, vs), ks, vs


def _finish_tables(lists, max_seqs, max_pages):
    tables = np.full((max_seqs, max_pages), -1, np.int32)
    counts = np.zeros(max_seqs, np.int32)
    for s, pages in enumerate(lists):
        tables[s, :len(pages)] = pages
        counts[s] = len(pages)
    return tables, counts


def _offsets(hist_len):
    off = np.zeros(len(hist_len), np.int64)
    if len(hist_len) > 1:
        off[1:] = np.cumsum(hist_len)[:-1]
    return off


def make(name: str, device: str | torch.device = "cpu", seed: int = 0, **kw) -> Workload:
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    return BUILDERS[name](gen, rng, dev, **kw)


def _layer_shapes(D, nq, nkv, d, F):
    shapes = [("w_qkv", ((nq + 2 * nkv) * d, D)), ("w_o", (D, nq * d))]
    if F:
        shapes += [("w_gu", (2 * F, D)), ("w_d", (D, F))]
    return shapes


def _tiny(gen, rng, dev, attention_only: bool = False, lens=(5, 17, 64, 100)):
    """Tiny fp32 layer: D 256, 4 q heads, 2 kv heads, d 64; four sequences of
    the given context lengths in a 16-page pool at random pages."""
    D, nq, nkv, d = 256, 4, 2, 64
    ws, sc = _weights(gen, dev, F32, _layer_shapes(D, nq, nkv, d, 0))
    lens = np.asarray(lens, np.int32)
    pages_needed = (lens + 31) // 32
    perm = rng.permutation(16)
    lists, o = [], 0
    for n in pages_needed:
        lists.append(perm[o:o + n].tolist()); o += n
    tables, counts = _finish_tables(lists, len(lens), 4)
    hist_len = lens if attention_only else lens - 1
    hk, hv, _, _ = _history(gen, dev, int(hist_len.sum()), nkv, d, F32)
    B = len(lens)
    x = torch.randn((B, D), generator=gen, device=dev)
    w = Workload("tiny-f32", D, nq, nkv, d, 0, F32, F32, F32, GEMV, 0, 2, 16, B, 4, tables, counts,
                 hist_len.astype(np.int32), _offsets(hist_len), hk, hv,
                 np.arange(B, dtype=np.int32), (lens - 1).astype(np.int32), x, ws, sc)
    if attention_only:
        w.q = torch.randn((B, nq, d), generator=gen, device=dev)
    return w


def _b1_06(gen, rng, dev, L: int = 2048, chunk: int = 2, family: int = GEMV):
    """0.6B-class layer at batch 1: D 1024, 16 q / 8 kv heads, d 128, F 3072,
    bf16; one sequence of L tokens in pages placed at random in a 256-page pool."""
    D, nq, nkv, d, F = 1024, 16, 8, 128, 3072
    ws, sc = _weights(gen, dev, BF16, _layer_shapes(D, nq, nkv, d, F))
    npg = (L + 31) // 32
    pool = max(256, npg)
    lists = [rng.permutation(pool)[:npg].tolist()]
    tables, counts = _finish_tables(lists, 1, npg)
    hist_len = np.asarray([L - 1], np.int32)
    hk, hv, _, _ = _history(gen, dev, L - 1, nkv, d, BF16)
    x = torch.randn((1, D), generator=gen, device=dev)
    return Workload("0.6b-b1-bf16", D, nq, nkv, d, F, BF16, BF16, BF16, family, 0, chunk, pool, 1,
                    npg, tables, counts, hist_len, _offsets(hist_len), hk, hv,
                    np.zeros(1, np.int32), np.asarray([L - 1], np.int32), x, ws, sc)


def _mixed_06(gen, rng, dev, n_decode: int = 512, chunk_rows: int = 256, chunk: int = 8,
              family: int = MFMA, long_max: int = 2662):
    """0.6B-class layer, mixed step: n_decode decode rows (80% with context
    U{100..200}, 20% U{1000..long_max}) plus `chunk_rows` rows of one 2,662-token
    prompt at positions 1024.. (a prefill chunk mixed into the step).  Pages of
    all sequences are a random permutation of a pool of exactly the pages needed."""
    D, nq, nkv, d, F = 1024, 16, 8, 128, 3072
    ws, sc = _weights(gen, dev, BF16, _layer_shapes(D, nq, nkv, d, F))
    n_long = int(round(0.2 * n_decode))
    is_long = np.zeros(n_decode, bool)
    is_long[rng.permutation(n_decode)[:n_long]] = True
    lens = np.where(is_long, rng.integers(1000, long_max + 1, n_decode),
                    rng.integers(100, 201, n_decode)).astype(np.int32)
    prompt = 2662
    c0 = 1024
    cap = [(int(L) + 31) // 32 for L in lens] + [(prompt + 31) // 32]
    total_pages = int(sum(cap))
    perm = rng.permutation(total_pages)
    lists, o = [], 0
    for n in cap:
        lists.append(perm[o:o + n].tolist()); o += n
    S = n_decode + 1
    max_pages = max(cap)
    tables, counts = _finish_tables(lists, S, max_pages)
    hist_len = np.concatenate([lens - 1, [c0]]).astype(np.int32)
    hk, hv, _, _ = _history(gen, dev, int(hist_len.sum()), nkv, d, BF16)
    seq = np.concatenate([np.arange(n_decode), np.full(chunk_rows, n_decode)]).astype(np.int32)
    pos = np.concatenate([lens - 1, c0 + np.arange(chunk_rows)]).astype(np.int32)
    B = seq.size
    x = torch.randn((B, D), generator=gen, device=dev)
    return Workload("0.6b-mixed-bf16", D, nq, nkv, d, F, BF16, BF16, BF16, family, 0, chunk,
                    total_pages, S, max_pages, tables, counts, hist_len, _offsets(hist_len), hk,
                    hv, seq, pos, x, ws, sc)


def _b768_7b(gen, rng, dev, n: int = 768, family: int = MFMA, chunk: int = 8,
             with_weights: bool = True):
    """7B-class layer, batch 768: D 3584, 28 q / 4 kv heads, d 128, F 18944,
    bf16.  Each sequence is a 128-token prompt plus g ~ U{1..128} generated
    tokens (context 128 + g); the first 90 prompt tokens (70%) are one prefix
    common to all sequences, whose two whole pages are shared physically
    through the block tables; 8 pages are reserved per sequence."""
    D, nq, nkv, d, F = 3584, 28, 4, 128, 18944
    ws, sc = ({}, {})
    if with_weights:
        ws, sc = _weights(gen, dev, BF16, _layer_shapes(D, nq, nkv, d, F))
    g = rng.integers(1, 129, n)
    lens = (128 + g).astype(np.int32)
    shared = 2
    private = 6
    num_pages = shared + n * private
    perm = rng.permutation(num_pages)
    shared_pages = perm[:shared].tolist()
    lists = [shared_pages + perm[shared + i * private: shared + (i + 1) * private].tolist()
             for i in range(n)]
    tables, counts = _finish_tables(lists, n, shared + private)
    hist_len = (lens - 1).astype(np.int32)
    total = int(hist_len.sum())
    hk, hv, _, _ = _history(gen, dev, total, nkv, d, BF16)
    # the 90-token prefix is the same content in every sequence
    off = _offsets(hist_len)
    for s in range(1, n):
        hk[off[s]:off[s] + 90] = hk[0:90]
        hv[off[s]:off[s] + 90] = hv[0:90]
    x = torch.randn((n, D), generator=gen, device=dev)
    return Workload("7b-b768-prefix-bf16", D, nq, nkv, d, F, BF16, BF16, BF16, family, 0, chunk,
                    num_pages, n, shared + private, tables, counts, hist_len, off, hk, hv,
                    np.arange(n, dtype=np.int32), (lens - 1).astype(np.int32), x, ws, sc,
                    notes="shared physical pages: 2 per sequence")


def _b4096_fp8(gen, rng, dev, n: int = 4096, L: int = 1024, family: int = MFMA_FP8,
               with_weights: bool = True):
    """7B-class layer, batch 4096, fp8: E4M3 weights (per-tensor scales) and KV
    (scales max|v| / 448 over the history), contexts of L tokens in 32-token
    pages placed by a random permutation of the whole pool.  The projections
    run as native fp8 matrix-core contractions (family 2) unless `family`
    says otherwise."""
    D, nq, nkv, d, F = 3584, 28, 4, 128, 18944
    ws, sc = ({}, {})
    if with_weights:
        ws, sc = _weights(gen, dev, FP8, _layer_shapes(D, nq, nkv, d, F))
    npg = (L + 31) // 32
    num_pages = n * npg
    perm = rng.permutation(num_pages)
    lists = [perm[i * npg:(i + 1) * npg].tolist() for i in range(n)]
    tables, counts = _finish_tables(lists, n, npg)
    hist_len = np.full(n, L - 1, np.int32)
    hk, hv, ks, vs = _history(gen, dev, int(hist_len.sum()), nkv, d, FP8)
    x = torch.randn((n, D), generator=gen, device=dev)
    return Workload("7b-b4096-fp8", D, nq, nkv, d, F, FP8, FP8, BF16, family, 1, npg, num_pages, n,
                    npg, tables, counts, hist_len, _offsets(hist_len), hk, hv,
                    np.arange(n, dtype=np.int32), np.full(n, L - 1, np.int32), x, ws, sc,
                    k_scale=ks, v_scale=vs)


def _prefill(gen, rng, dev, layer: str = "7b", p0: int = 1024, n: int = 256, prompt: int = 2662,
             chunk: int = 8, family: int = MFMA):
    """One prompt of `prompt` tokens (the 2,662-token request of "GPU inference
    engine engineering", section "Batching without running out of cache")
    prefilled in chunks of n = 256 tokens ("13.4x faster prefill in 256-token
    chunks"): the rows are the chunk's positions p0 .. p0 + n - 1 of sequence
    0; the pool holds the first p0 tokens as history; all the prompt's pages
    are reserved, placed at random; bf16 weights and KV of the named layer."""
    D, nq, nkv, d, F = {"7b": (3584, 28, 4, 128, 18944), "0.6b": (1024, 16, 8, 128, 3072)}[layer]
    ws, sc = _weights(gen, dev, BF16, _layer_shapes(D, nq, nkv, d, F))
    npg = (prompt + 31) // 32
    lists = [rng.permutation(npg).tolist()]
    tables, counts = _finish_tables(lists, 1, npg)
    hist_len = np.asarray([p0], np.int32)
    hk, hv, _, _ = _history(gen, dev, p0, nkv, d, BF16)
    x = torch.randn((n, D), generator=gen, device=dev)
    return Workload(f"prefill-{layer}-bf16", D, nq, nkv, d, F, BF16, BF16, BF16, family, 0, chunk, npg, 1, npg,
                    tables, counts, hist_len, _offsets(hist_len), hk, hv, np.zeros(n, np.int32),
                    (p0 + np.arange(n)).astype(np.int32), x, ws, sc)


def _attn_case(gen, rng, dev, n_q=4, n_kv=2, d=128, kv_dtype=BF16, lens=(1, 31, 32, 33, 64, 65, 100),
               append=True, chunk=2, extra_pages=3, shared_first_page=False):
    """Attention-only case: one row per sequence at position len - 1; the pool
    holds len - 1 positions (append) or all len positions; pages at random,
    `extra_pages` spare pages per sequence reserved in the tables."""
    lens = np.asarray(lens, np.int32)
    S = len(lens)
    need = (lens + 31) // 32
    reserve = need + extra_pages
    num_pages = int(reserve.sum()) + 3
    perm = rng.permutation(num_pages)
    lists, o = [], 0
    for n in reserve:
        lists.append(perm[o:o + n].tolist()); o += n
    if shared_first_page and S > 1:
        for s in range(1, S):
            if lens[s] > 32 and lens[0] >= 32:
                lists[s][0] = lists[0][0]
    max_pages = int(reserve.max())
    tables, counts = _finish_tables(lists, S, max_pages)
    hist_len = (lens - 1 if append else lens).astype(np.int32)
    hk, hv, ks, vs = _history(gen, dev, int(hist_len.sum()), n_kv, d, kv_dtype)
    off = _offsets(hist_len)
    if shared_first_page:
        for s in range(1, S):
            if lens[s] > 32 and lens[0] >= 32:
                hk[off[s]:off[s] + 32] = hk[off[0]:off[0] + 32]
                hv[off[s]:off[s] + 32] = hv[off[0]:off[0] + 32]
    qd = F32 if kv_dtype == F32 else BF16
    x = torch.zeros((S, 64), device=dev)
    w = Workload(f"attn-{['f32', 'bf16', 'fp8'][kv_dtype]}-g{n_q // n_kv}-d{d}", 64, n_q, n_kv, d, 0, qd,
                 kv_dtype, qd, GEMV, 0, chunk, num_pages, S, max_pages, tables, counts, hist_len, off, hk, hv,
                 np.arange(S, dtype=np.int32), (lens - 1).astype(np.int32), x, k_scale=ks, v_scale=vs)
    w.q = encode(torch.randn((S, n_q, d), generator=gen, device=dev), qd)
    if append:
        w.k_new = encode(torch.randn((S, n_kv, d), generator=gen, device=dev), qd)
        w.v_new = encode(torch.randn((S, n_kv, d), generator=gen, device=dev), qd)
    return w


BUILDERS = {
    "attn": _attn_case,
    "tiny-f32": _tiny,
    "0.6b-b1-bf16": _b1_06,
    "0.6b-mixed-bf16": _mixed_06,
    "7b-b768-prefix-bf16": _b768_7b,
    "7b-b4096-fp8": _b4096_fp8,
    "prefill-chunk": _prefill,
}


def layer_dict(w: Workload) -> dict:
    """The layer description the oracle takes (codes as numpy arrays)."""
    return dict(hidden=w.hidden, n_q=w.n_q, n_kv=w.n_kv, head_dim=w.head_dim, ffn=w.ffn,
                w_dtype=w.w_dtype,
                w_qkv=to_numpy_codes(w.weights["w_qkv"], w.w_dtype),
                w_o=to_numpy_codes(w.weights["w_o"], w.w_dtype),
                w_gu=to_numpy_codes(w.weights["w_gu"], w.w_dtype) if w.ffn else None,
                w_d=to_numpy_codes(w.weights["w_d"], w.w_dtype) if w.ffn else None,
                s_qkv=w.scales.get("w_qkv", 1.0), s_o=w.scales.get("w_o", 1.0),
                s_gu=w.scales.get("w_gu", 1.0), s_d=w.scales.get("w_d", 1.0),
                act_dtype=w.act_dtype, act_fp8=w.act_fp8, kv_dtype=w.kv_dtype,
                k_scale=w.k_scale, v_scale=w.v_scale, norm=w.norm, rope=w.rope,
                norm_eps=w.norm_eps, rope_base=w.rope_base)


def with_norm_rope(w: Workload, x_std: float = 3.0) -> Workload:
    """The same workload with both norms and rotary positions switched on.
    The weights stand for weights with the norm gains already folded in (a
    random gain times a random weight is another random weight), and x is
    rescaled to standard deviation x_std so that 1/rms is far from 1."""
    w.norm = True
    w.rope = True
    w.x = w.x * x_std
    w.name += "+norm+rope"
    return w


def history_lists(w: Workload, seqs=None):
    """Per-sequence numpy history code arrays (all sequences, or only `seqs`;
    the others get empty histories)."""
    want = None if seqs is None else set(int(s) for s in seqs)
    hk, hv = [], []
    d0 = np.zeros((0, w.n_kv, w.head_dim), {F32: np.float32, BF16: np.uint16, FP8: np.uint8}[w.kv_dtype])
    for s in range(len(w.hist_len)):
        if want is not None and s not in want:
            hk.append(d0); hv.append(d0); continue
        o, L = int(w.hist_off[s]), int(w.hist_len[s])
        hk.append(to_numpy_codes(w.hist_k[o:o + L], w.kv_dtype))
        hv.append(to_numpy_codes(w.hist_v[o:o + L], w.kv_dtype))
    return hk, hv


# ----------------------------------------------------------------------------- output head
# A tied embedding of 151,936 rows by 2,048 bf16 columns is 593.5 MiB and 28
# of its rows are 112 KiB: the full-head and candidate-head read sizes of the
# grammar-bounded output layer ("GPU inference engine engineering", headline
# figure "Grammar-bounded output", at most 28 edges per trie node).
HEAD_VOCAB, HEAD_HIDDEN, HEAD_MAX_CAND = 151936, 2048, 28


def head_candidates(n: int, vocab: int, max_cand: int = HEAD_MAX_CAND, seed: int = 0):
    """Per-row candidate lists shaped like a trie node's outgoing edges:
    1 .. max_cand distinct rows of the vocabulary (count uniform), in random
    order; unused slots hold -1.  Returns (cand int32 [n][max_cand],
    n_cand int32 [n]) as numpy arrays."""
    rng = np.random.default_rng(seed)
    cand = np.full((n, max_cand), -1, np.int32)
    n_cand = rng.integers(1, max_cand + 1, size=n).astype(np.int32)
    for r in range(n):
        cand[r, :n_cand[r]] = rng.choice(vocab, size=n_cand[r], replace=False)
    return cand, n_cand
