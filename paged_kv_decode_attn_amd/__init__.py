"""Python binding of libpkd (paged-KV decode step for MI355X / gfx950).

Argument marshalling only: every function forwards to the C ABI of the same
name (include/pkd.h) with raw device pointers and a HIP stream taken from
torch.  torch supplies device memory and streams; all arithmetic runs in the
library's HIP kernels.  Importing the package loads libpkd.so and fails loudly
if it has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that the library then shares

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkd.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
FAMILY_GEMV, FAMILY_MFMA, FAMILY_MFMA_FP8, FAMILY_GEMV_MFMA = 0, 1, 2, 3
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "out of memory", 4: "out of bounds",
          5: "duplicate page", 6: "device error", 7: "invalid row"}


class PkdError(RuntimeError):
    def __init__(self, status: int, needed: int, available: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail} (needed={needed}, available={available})")
        self.status = status
        self.needed = needed
        self.available = available
        self.detail = detail


# ------------------------------------------------------------------ C structs
class pkd_error(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("needed", ctypes.c_int64), ("available", ctypes.c_int64),
                ("detail", ctypes.c_char * 192)]


class pkd_pool_desc(ctypes.Structure):
    _fields_ = [("num_pages", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("max_seqs", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("attn_chunk_pages", ctypes.c_int32)]


class pkd_pool_info(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("pages_offset", ctypes.c_size_t),
                ("block_bytes", ctypes.c_size_t), ("table_offset", ctypes.c_size_t),
                ("counts_offset", ctypes.c_size_t), ("error_offset", ctypes.c_size_t),
                ("shared_pages", ctypes.c_int64)]


ROWS_DISTINCT_SEQS = 1


class pkd_rows(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("n", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class pkd_matrix(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("family", ctypes.c_int32),
                ("k_splits", ctypes.c_int32)]


class pkd_epilogue(ctypes.Structure):
    _fields_ = [("out_dtype", ctypes.c_int32), ("residual", ctypes.c_void_p),
                ("silu_pair", ctypes.c_int32), ("y_bf16", ctypes.c_void_p),
                ("row_scale", ctypes.c_void_p), ("rope_cs", ctypes.c_void_p),
                ("rope_cols", ctypes.c_int32), ("rope_head_dim", ctypes.c_int32)]


class pkd_layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("w_qkv", pkd_matrix), ("w_o", pkd_matrix), ("w_gate_up", pkd_matrix),
                ("w_down", pkd_matrix), ("act_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("rope_base", ctypes.c_float)]


LAYER_NORM, LAYER_ROPE = 1, 2


EXPORTS = ["pkd_pool_bytes", "kv_pool_create", "kv_pool_destroy", "pkd_pool_info_get", "block_table_set",
           "pkd_pool_check", "pkd_attn_workspace_bytes", "paged_attn_decode", "pkd_attn_noalloc_scratch_bytes",
           "paged_attn_decode_noalloc", "pkd_gemv_workspace_bytes",
           "pkd_suggest_k_splits", "gemv_rows", "gemv_gather_rows", "rms_norm_factor", "rope_table",
           "pkd_step_workspace_bytes", "decode_step", "pkd_status_string", "pkd_version"]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"libpkd.so is not built ({path}); run paged_kv_decode_attn_amd/build.py "
                           "or __graft_entry__.build()")
    L = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    E = ctypes.POINTER(pkd_error)
    sig = {
        "pkd_pool_bytes": (SZ, [ctypes.POINTER(pkd_pool_desc)]),
        "kv_pool_create": (I32, [ctypes.POINTER(pkd_pool_desc), P, SZ, P, ctypes.POINTER(P), E]),
        "kv_pool_destroy": (I32, [P]),
        "pkd_pool_info_get": (I32, [P, ctypes.POINTER(pkd_pool_info)]),
        "block_table_set": (I32, [P, I32, I32, P, P, P, E]),
        "pkd_pool_check": (I32, [P, P, E]),
        "pkd_attn_workspace_bytes": (SZ, [P, I32, I32]),
        "paged_attn_decode": (I32, [P, ctypes.POINTER(pkd_rows), I32, P, P, P, P, I32, P, SZ, P, E]),
        "pkd_attn_noalloc_scratch_bytes": (SZ, []),
        "paged_attn_decode_noalloc": (I32, [P, ctypes.POINTER(pkd_rows), I32, P, P, P, P, I32, P, E]),
        "pkd_gemv_workspace_bytes": (SZ, [ctypes.POINTER(pkd_matrix), I32]),
        "pkd_suggest_k_splits": (I32, [I32, I32, I32, I32]),
        "gemv_rows": (I32, [ctypes.POINTER(pkd_matrix), P, I32, I32, P, ctypes.POINTER(pkd_epilogue), P, SZ,
                            P, E]),
        "gemv_gather_rows": (I32, [ctypes.POINTER(pkd_matrix), P, I32, I32, P, P, I32, P, P, E]),
        "rms_norm_factor": (I32, [P, I32, I32, ctypes.c_float, P, P, P, E]),
        "rope_table": (I32, [P, I32, I32, ctypes.c_float, P, P, E]),
        "pkd_step_workspace_bytes": (SZ, [ctypes.POINTER(pkd_layer), P, I32]),
        "decode_step": (I32, [ctypes.POINTER(pkd_layer), P, ctypes.POINTER(pkd_rows), P, P, P, SZ, P, E]),
        "pkd_status_string": (ctypes.c_char_p, [I32]),
        "pkd_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def _check(status: int, err: pkd_error) -> None:
    if status != 0:
        raise PkdError(status, err.needed, err.available, err.detail.decode(errors="replace"))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ pool
def pkd_pool_bytes(desc: pkd_pool_desc) -> int:
    return lib().pkd_pool_bytes(ctypes.byref(desc))


def kv_pool_create(desc: pkd_pool_desc, dev_mem: torch.Tensor, stream=None) -> ctypes.c_void_p:
    err = pkd_error()
    h = ctypes.c_void_p()
    _check(lib().kv_pool_create(ctypes.byref(desc), _ptr(dev_mem), dev_mem.numel() * dev_mem.element_size(),
                                _stream(stream), ctypes.byref(h), ctypes.byref(err)), err)
    return h


def kv_pool_destroy(pool) -> None:
    lib().kv_pool_destroy(pool)


def pkd_pool_info_get(pool) -> pkd_pool_info:
    info = pkd_pool_info()
    if lib().pkd_pool_info_get(pool, ctypes.byref(info)) != 0:
        raise PkdError(1, 0, 0, "pkd_pool_info_get")
    return info


def block_table_set(pool, first_seq: int, pages, counts, stream=None) -> None:
    """pages: host int32 array [n_seqs][max_pages_per_seq]; counts: host int32 [n_seqs]."""
    import numpy as np
    pages = np.ascontiguousarray(pages, dtype=np.int32)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    err = pkd_error()
    _check(lib().block_table_set(pool, first_seq, counts.size, pages.ctypes.data, counts.ctypes.data,
                                 _stream(stream), ctypes.byref(err)), err)


def pkd_pool_check(pool, stream=None) -> None:
    err = pkd_error()
    _check(lib().pkd_pool_check(pool, _stream(stream), ctypes.byref(err)), err)


# ------------------------------------------------------------------ attention
def make_rows(seq: torch.Tensor, pos: torch.Tensor, distinct: bool = False) -> pkd_rows:
    r = pkd_rows(_ptr(seq), _ptr(pos), int(seq.numel()), ROWS_DISTINCT_SEQS if distinct else 0)
    r._keep = (seq, pos)  # the struct holds raw pointers: keep the tensors alive with it
    return r


def pkd_attn_workspace_bytes(pool, n_q_heads: int, max_rows: int) -> int:
    return lib().pkd_attn_workspace_bytes(pool, n_q_heads, max_rows)


def paged_attn_decode(pool, rows: pkd_rows, n_q_heads: int, q, k_new, v_new, out, out_dtype: int, ws,
                      stream=None) -> None:
    err = pkd_error()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().paged_attn_decode(pool, ctypes.byref(rows), n_q_heads, _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(out), out_dtype, _ptr(ws), ws_bytes, _stream(stream),
                                   ctypes.byref(err)), err)


def pkd_attn_noalloc_scratch_bytes() -> int:
    return lib().pkd_attn_noalloc_scratch_bytes()


def paged_attn_decode_noalloc(pool, rows: pkd_rows, n_q_heads: int, q, k_new, v_new, out, out_dtype: int,
                              stream=None) -> None:
    """paged_attn_decode with the library's fixed per-GPU scratch instead of a workspace."""
    err = pkd_error()
    _check(lib().paged_attn_decode_noalloc(pool, ctypes.byref(rows), n_q_heads, _ptr(q), _ptr(k_new), _ptr(v_new),
                                           _ptr(out), out_dtype, _stream(stream), ctypes.byref(err)), err)


# ------------------------------------------------------------------ projections
def make_matrix(data: torch.Tensor, rows: int, cols: int, dtype: int, scale: float = 1.0,
                family: int = FAMILY_GEMV, k_splits: int = 1) -> pkd_matrix:
    m = pkd_matrix(_ptr(data), rows, cols, dtype, scale, family, k_splits)
    m._keep = data  # the struct holds a raw pointer: keep the tensor alive with it
    return m


def pkd_gemv_workspace_bytes(W: pkd_matrix, max_rows: int) -> int:
    return lib().pkd_gemv_workspace_bytes(ctypes.byref(W), max_rows)


def pkd_suggest_k_splits(rows: int, cols: int, family: int, typical_rows: int) -> int:
    return lib().pkd_suggest_k_splits(rows, cols, family, typical_rows)


def gemv_rows(W: pkd_matrix, x, x_dtype: int, n_rows: int, y, out_dtype: int = F32, residual=None,
              silu_pair: bool = False, y_bf16=None, ws=None, stream=None, row_scale=None, rope_cs=None,
              rope_cols: int = 0, rope_head_dim: int = 0) -> None:
    ep = pkd_epilogue(out_dtype, _ptr(residual), 1 if silu_pair else 0, _ptr(y_bf16), _ptr(row_scale),
                      _ptr(rope_cs), rope_cols, rope_head_dim)
    err = pkd_error()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gemv_rows(ctypes.byref(W), _ptr(x), x_dtype, n_rows, _ptr(y), ctypes.byref(ep), _ptr(ws),
                           ws_bytes, _stream(stream), ctypes.byref(err)), err)


def gemv_gather_rows(W: pkd_matrix, x, x_dtype: int, n_rows: int, cand, n_cand, max_cand: int, y,
                     stream=None) -> None:
    """y[r][c] = W[cand[r][c]] . x[r] for c < n_cand[r] (f32 logits)."""
    err = pkd_error()
    _check(lib().gemv_gather_rows(ctypes.byref(W), _ptr(x), x_dtype, n_rows, _ptr(cand), _ptr(n_cand), max_cand,
                                  _ptr(y), _stream(stream), ctypes.byref(err)), err)


def rms_norm_factor(x, n_rows: int, cols: int, eps: float, inv_rms, x_bf16=None, stream=None) -> None:
    """inv_rms[r] = 1 / sqrt(mean(x[r]^2) + eps); optionally x rounded to bf16."""
    err = pkd_error()
    _check(lib().rms_norm_factor(_ptr(x), n_rows, cols, eps, _ptr(inv_rms), _ptr(x_bf16), _stream(stream),
                                 ctypes.byref(err)), err)


def rope_table(pos, n_rows: int, head_dim: int, base: float, cs, stream=None) -> None:
    """cs[r][i] = (cos, sin) of pos[r] * base^(-2i / head_dim)."""
    err = pkd_error()
    _check(lib().rope_table(_ptr(pos), n_rows, head_dim, base, _ptr(cs), _stream(stream), ctypes.byref(err)), err)


# ------------------------------------------------------------------ decode step
def pkd_step_workspace_bytes(layer: pkd_layer, pool, max_rows: int) -> int:
    return lib().pkd_step_workspace_bytes(ctypes.byref(layer), pool, max_rows)


def decode_step(layer: pkd_layer, pool, rows: pkd_rows, x, y, ws, stream=None) -> None:
    err = pkd_error()
    _check(lib().decode_step(ctypes.byref(layer), pool, ctypes.byref(rows), _ptr(x), _ptr(y), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream), ctypes.byref(err)), err)


def pkd_version() -> str:
    return lib().pkd_version().decode()
