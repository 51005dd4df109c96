"""Builds GPU-side objects (pool, weights, rows) for a Workload and runs the
library through its Python binding.  Test and benchmark infrastructure."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_decode_attn_amd as pkd
import workloads as wl

DEV = "cuda"


def rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max over rows of max_j |got - want| / max_j |want| (per row, per tensor)."""
    got = np.asarray(got, np.float64).reshape(got.shape[0], -1)
    want = np.asarray(want, np.float64).reshape(want.shape[0], -1)
    num = np.abs(got - want).max(axis=1)
    den = np.abs(want).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if got.size else 0.0


def values(t: torch.Tensor, dtype: int) -> np.ndarray:
    """Device tensor of stored codes (f32, bf16 bits as int16/uint16) -> float64 numpy."""
    t = t.detach()
    if dtype == wl.BF16:
        return t.view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


class GpuPool:
    """pad: bytes of guard memory (filled with 0xA5) allocated before and after
    the pool's buffer, so that tests can check that nothing outside the pool
    was written."""

    def __init__(self, w: wl.Workload, chunk_pages: int | None = None, poison: bool = True, pad: int = 0):
        self.w = w
        chunk = w.attn_chunk_pages if chunk_pages is None else chunk_pages
        self.desc = pkd.pkd_pool_desc(w.num_pages, 32, w.n_kv, w.head_dim, w.kv_dtype, w.k_scale,
                                      w.v_scale, w.max_seqs, w.max_pages_per_seq, chunk)
        nbytes = pkd.pkd_pool_bytes(self.desc)
        assert nbytes > 0
        pad = (pad + 255) // 256 * 256
        self.mem = torch.empty(nbytes + 2 * pad + 256, dtype=torch.uint8, device=DEV)
        if pad:
            self.mem.fill_(0xA5)
        off = (-self.mem.data_ptr()) % 256 + pad
        self.pad = pad
        self.buf = self.mem[off:off + nbytes]
        self.handle = pkd.kv_pool_create(self.desc, self.buf)
        self.info = pkd.pkd_pool_info_get(self.handle)
        npb = w.num_pages * w.n_kv * 2 * self.info.block_bytes
        pages = self.buf[self.info.pages_offset:self.info.pages_offset + npb]
        hk = w.hist_k.to(DEV)
        hv = w.hist_v.to(DEV)
        wl.fill_pool_pages(pages, w.num_pages, w.n_kv, w.head_dim, w.kv_dtype, w.tables, w.counts, hk, hv,
                           w.hist_off, w.hist_len, poison=poison)
        del hk, hv
        pkd.block_table_set(self.handle, 0, w.tables, w.counts)
        torch.cuda.synchronize()

    def guard_intact(self) -> bool:
        """The guard bytes around the pool still hold their fill."""
        off = self.buf.data_ptr() - self.mem.data_ptr()
        before, after = self.mem[:off], self.mem[off + self.buf.numel():]
        return bool((before[off - self.pad:] == 0xA5).all()) and bool((after[:self.pad] == 0xA5).all())

    def table_entries(self) -> torch.Tensor:
        """The device copy of the block tables, int32 [max_seqs][max_pages_per_seq]."""
        n = self.w.max_seqs * self.w.max_pages_per_seq
        return self.buf[self.info.table_offset:self.info.table_offset + 4 * n].view(torch.int32).view(
            self.w.max_seqs, self.w.max_pages_per_seq)

    def pages_bytes(self) -> torch.Tensor:
        w = self.w
        npb = w.num_pages * w.n_kv * 2 * self.info.block_bytes
        return self.buf[self.info.pages_offset:self.info.pages_offset + npb]

    def __del__(self):
        try:
            pkd.kv_pool_destroy(self.handle)
        except Exception:
            pass


def aligned_empty(nbytes: int) -> torch.Tensor:
    mem = torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=DEV)
    off = (-mem.data_ptr()) % 256
    return mem[off:off + max(nbytes, 1)]


def rows_tensors(seq, pos):
    s = torch.as_tensor(np.asarray(seq, np.int32), device=DEV)
    p = torch.as_tensor(np.asarray(pos, np.int32), device=DEV)
    return s, p


def run_attention(pool: GpuPool, seq, pos, q: torch.Tensor, k_new=None, v_new=None,
                  out_dtype: int = wl.F32, distinct: bool = False) -> torch.Tensor:
    w = pool.w
    s, p = rows_tensors(seq, pos)
    n = s.numel()
    rows = pkd.make_rows(s, p, distinct)
    ws = aligned_empty(pkd.pkd_attn_workspace_bytes(pool.handle, w.n_q, n))
    out = torch.empty((n, w.n_q, w.head_dim), dtype=torch.float32 if out_dtype == wl.F32 else torch.int16,
                      device=DEV)
    pkd.paged_attn_decode(pool.handle, rows, w.n_q, q, k_new, v_new, out, out_dtype, ws)
    torch.cuda.synchronize()
    return out


class GpuLayer:
    """Device copy of a workload's layer.  batch_hint: the batch the engine is
    built for; matrix-core matrices then take the library's suggested K split
    (fixed for the life of the layer, so results stay batch invariant)."""

    def __init__(self, w: wl.Workload, family: int | None = None, batch_hint: int | None = None):
        self.w = w
        fam = w.family if family is None else family
        self.tensors = {k: v.to(DEV).contiguous() for k, v in w.weights.items()}
        D, nq, nkv, d, F = w.hidden, w.n_q, w.n_kv, w.head_dim, w.ffn
        nqkv = (nq + 2 * nkv) * d

        def M(name, rows, cols):
            if name not in self.tensors:
                return pkd.pkd_matrix()
            S = pkd.pkd_suggest_k_splits(rows, cols, fam, batch_hint) if batch_hint else 1
            return pkd.make_matrix(self.tensors[name], rows, cols, w.w_dtype, w.scales.get(name, 1.0), fam, S)
        flags = (pkd.LAYER_NORM if w.norm else 0) | (pkd.LAYER_ROPE if w.rope else 0)
        self.layer = pkd.pkd_layer(D, nq, nkv, d, F, M("w_qkv", nqkv, D), M("w_o", D, nq * d),
                                   M("w_gu", 2 * F, D), M("w_d", D, F), w.act_dtype, flags, w.norm_eps,
                                   w.rope_base)

    def step(self, pool: GpuPool, seq, pos, x: torch.Tensor, ws: torch.Tensor | None = None):
        s, p = rows_tensors(seq, pos)
        n = s.numel()
        distinct = len(set(np.asarray(seq).tolist())) == n  # pure decode batch: append fused into attention
        rows = pkd.make_rows(s, p, distinct)
        if ws is None:
            ws = aligned_empty(pkd.pkd_step_workspace_bytes(self.layer, pool.handle, n))
        y = torch.empty((n, self.w.hidden), dtype=torch.float32, device=DEV)
        pkd.decode_step(self.layer, pool.handle, rows, x.to(DEV).contiguous(), y, ws)
        torch.cuda.synchronize()
        return y
