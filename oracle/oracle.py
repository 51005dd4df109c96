"""ctypes wrapper of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg.  The product path never imports it.
It shares no code with the HIP library; see oracle.c for what each function
computes and which passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16, FP8 = 0, 1, 2
NORM, ROPE = 1, 2
_NP = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}


def build(force: bool = False) -> str:
    """Compiles liboracle.so with gcc (plain C, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        L.orc_threads.restype = ctypes.c_int
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_round.restype = ctypes.c_uint16
        L.orc_bf16_round.argtypes = [ctypes.c_double]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_round_sat.restype = ctypes.c_uint8
        L.orc_e4m3_round_sat.argtypes = [ctypes.c_double]
        for name in ("orc_bf16_round_array", "orc_bf16_value_array", "orc_e4m3_round_array",
                     "orc_e4m3_value_array"):
            getattr(L, name).argtypes = [P, P, ctypes.c_int64]
            getattr(L, name).restype = None
        L.orc_act_quant.argtypes = [P, ctypes.c_int64, P, P]
        L.orc_act_quant.restype = None
        L.orc_matvec_rows.argtypes = [ctypes.c_int, P, ctypes.c_double, ctypes.c_int,
                                      ctypes.c_int, P, ctypes.c_int, P]
        L.orc_matvec_rows.restype = None
        L.orc_matvec_gathered.argtypes = [ctypes.c_int, P, ctypes.c_double, ctypes.c_int, ctypes.c_int, P,
                                          ctypes.c_int, P, ctypes.c_int, P, P]
        L.orc_matvec_gathered.restype = None
        L.orc_inv_rms_rows.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_double, P]
        L.orc_inv_rms_rows.restype = None
        L.orc_rope_rows.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_double]
        L.orc_rope_rows.restype = None
        L.orc_gather_history.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P,
                                         ctypes.c_int, ctypes.c_int, P, P]
        L.orc_gather_history.restype = ctypes.c_int
        L.orc_attention.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, P, P, P, P]
        L.orc_attention.restype = ctypes.c_int
        L.orc_decode_step.argtypes = [P, P, ctypes.c_int, P, P, P, P]
        L.orc_decode_step.restype = ctypes.c_int
        _lib = L
    return _lib


def threads() -> int:
    return lib().orc_threads()


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


# ---------------------------------------------------------------- codecs
def bf16_round(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_round_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_value(c) -> np.ndarray:
    c = _c(c, np.uint16)
    out = np.empty(c.shape, np.float64)
    lib().orc_bf16_value_array(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_round(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_round_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_value(c) -> np.ndarray:
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_value_array(_ptr(c), _ptr(out), c.size)
    return out


def act_quant(z) -> tuple[np.ndarray, float]:
    z = _c(z, np.float64).reshape(-1)
    codes = np.empty(z.shape, np.uint8)
    s = np.zeros(1, np.float32)
    lib().orc_act_quant(_ptr(z), z.size, _ptr(codes), _ptr(s))
    return codes, float(s[0])


def code_values(codes: np.ndarray, dtype: int, scale: float = 1.0) -> np.ndarray:
    if dtype == F32:
        return np.asarray(codes, np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_value(codes)
    return e4m3_value(codes) * float(scale)


# ---------------------------------------------------------------- matvec
def matvec_rows(dtype: int, W: np.ndarray, scale: float, X: np.ndarray) -> np.ndarray:
    """Y[r][j] = sum_k W[j][k] * scale * X[r][k] in fp64."""
    W = _c(W, _NP[dtype])
    X = _c(X, np.float64)
    rows, cols = W.shape
    X2 = X.reshape(-1, cols)
    Y = np.empty((X2.shape[0], rows), np.float64)
    lib().orc_matvec_rows(dtype, _ptr(W), float(scale), rows, cols, _ptr(X2), X2.shape[0], _ptr(Y))
    return Y


def matvec_gathered(dtype: int, W: np.ndarray, scale: float, X: np.ndarray, cand: np.ndarray,
                    n_cand: np.ndarray, fill: float = 0.0) -> np.ndarray:
    """Y[r][c] = sum_k W[cand[r][c]][k] * scale * X[r][k] in fp64 for
    c < clamp(n_cand[r], 0, max_cand); NaN for an index outside the matrix;
    `fill` elsewhere."""
    W = _c(W, _NP[dtype])
    X = _c(X, np.float64)
    rows, cols = W.shape
    X2 = X.reshape(-1, cols)
    cand = _c(cand, np.int32)
    n = X2.shape[0]
    cand = cand.reshape(n, -1)
    n_cand = _c(n_cand, np.int32)
    Y = np.full((n, cand.shape[1]), fill, np.float64)
    lib().orc_matvec_gathered(dtype, _ptr(W), float(scale), rows, cols, _ptr(X2), n, _ptr(cand),
                              cand.shape[1], _ptr(n_cand), _ptr(Y))
    return Y


def inv_rms_rows(Z: np.ndarray, eps: float) -> np.ndarray:
    """1 / sqrt(mean(z^2) + eps) per row of Z, in fp64."""
    Z = _c(Z, np.float64)
    Z2 = Z.reshape(Z.shape[0], -1)
    out = np.empty(Z2.shape[0], np.float64)
    lib().orc_inv_rms_rows(_ptr(Z2), Z2.shape[0], Z2.shape[1], float(eps), _ptr(out))
    return out


def rope_rows(V: np.ndarray, n_heads: int, hd: int, pos, base: float) -> np.ndarray:
    """Rotary positions on rows of V [n][n_heads * hd] (consecutive pairs), fp64."""
    V = np.array(V, dtype=np.float64, order="C", copy=True).reshape(-1, n_heads * hd)
    pos = _c(pos, np.int32)
    lib().orc_rope_rows(_ptr(V), V.shape[0], n_heads, hd, _ptr(pos), float(base))
    return V


# ---------------------------------------------------------------- structs
class _Geom(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


class _Hist(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("hist_off", ctypes.c_void_p),
                ("hist_len", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("w_qkv", ctypes.c_void_p),
                ("w_o", ctypes.c_void_p), ("w_gu", ctypes.c_void_p), ("w_d", ctypes.c_void_p),
                ("s_qkv", ctypes.c_double), ("s_o", ctypes.c_double), ("s_gu", ctypes.c_double),
                ("s_d", ctypes.c_double), ("act_dtype", ctypes.c_int32),
                ("act_fp8", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("flags", ctypes.c_int32), ("norm_eps", ctypes.c_double), ("rope_base", ctypes.c_double)]


class _Out(ctypes.Structure):
    _fields_ = [("qkv", ctypes.c_void_p), ("attn", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("a", ctypes.c_void_p), ("y", ctypes.c_void_p), ("qkv_raw", ctypes.c_void_p),
                ("attn_raw", ctypes.c_void_p), ("a_raw", ctypes.c_void_p)]


class History:
    """Per-sequence contiguous KV history: hist_k[s] is [len_s][n_kv][d] codes."""

    def __init__(self, hist_k: list, hist_v: list, kv_dtype: int, n_kv: int, d: int):
        self.kv_dtype = kv_dtype
        lens = [int(k.shape[0]) for k in hist_k]
        self.hist_len = np.asarray(lens, np.int32)
        self.hist_off = np.zeros(len(lens), np.int64)
        if lens:
            self.hist_off[1:] = np.cumsum(lens)[:-1]
        dt = _NP[kv_dtype]
        shape = (max(1, sum(lens)), n_kv, d)
        self.k = np.zeros(shape, dt)
        self.v = np.zeros(shape, dt)
        for s, (k, v) in enumerate(zip(hist_k, hist_v)):
            o = int(self.hist_off[s])
            self.k[o:o + lens[s]] = k
            self.v[o:o + lens[s]] = v

    def struct(self) -> _Hist:
        return _Hist(len(self.hist_len), _ptr(self.hist_off), _ptr(self.hist_len), _ptr(self.k),
                     _ptr(self.v))


def attention(n_q: int, n_kv: int, d: int, kv_dtype: int, k_scale: float, v_scale: float,
              hist: History, seq, pos, q_dtype: int, q, k_new=None, v_new=None) -> np.ndarray:
    seq = _c(seq, np.int32)
    pos = _c(pos, np.int32)
    n = seq.size
    q = _c(q, _NP[q_dtype])
    k_new = None if k_new is None else _c(k_new, _NP[q_dtype])
    v_new = None if v_new is None else _c(v_new, _NP[q_dtype])
    out = np.empty((n, n_q, d), np.float64)
    g = _Geom(n_q, n_kv, d, kv_dtype, k_scale, v_scale)
    h = hist.struct()
    rc = lib().orc_attention(ctypes.byref(g), ctypes.byref(h), n, _ptr(seq), _ptr(pos), q_dtype,
                             _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out))
    if rc != 0:
        raise ValueError("oracle attention refused the rows (bad row or gap in a sequence)")
    return out


def gather_history(pages: np.ndarray, n_kv: int, d: int, kv_dtype: int, table_row, length: int):
    """Reads `length` positions of one sequence out of a host copy of the pool's
    page region, through its block-table row."""
    pages = _c(pages, np.uint8)
    table_row = _c(table_row, np.int32)
    dt = _NP[kv_dtype]
    k = np.zeros((length, n_kv, d), dt)
    v = np.zeros((length, n_kv, d), dt)
    rc = lib().orc_gather_history(_ptr(pages), n_kv, d, kv_dtype, _ptr(table_row),
                                  table_row.size, length, _ptr(k), _ptr(v))
    if rc != 0:
        raise ValueError("gather_history: position past the block table")
    return k, v


def decode_step(layer: dict, hist: History, seq, pos, x, raw: bool = False) -> dict:
    """layer: hidden, n_q, n_kv, head_dim, ffn, w_dtype, w_qkv, w_o, w_gu, w_d (code
    arrays), s_qkv, s_o, s_gu, s_d, act_dtype, act_fp8, kv_dtype, k_scale, v_scale;
    optional norm (bool, gains already folded into w_qkv / w_gu), norm_eps,
    rope (bool), rope_base.  raw: also return qkv_raw, attn_raw, a_raw, the
    stored stages before their rounding to the activation dtype."""
    seq = _c(seq, np.int32)
    pos = _c(pos, np.int32)
    x = _c(x, np.float32)
    n = seq.size
    D, d, nq, nkv, F = (layer[k] for k in ("hidden", "head_dim", "n_q", "n_kv", "ffn"))
    wdt = _NP[layer["w_dtype"]]
    keep = [_c(layer[k], wdt) if layer.get(k) is not None else None
            for k in ("w_qkv", "w_o", "w_gu", "w_d")]
    L = _Layer(D, nq, nkv, d, F, layer["w_dtype"], *[_ptr(w) for w in keep],
               float(layer.get("s_qkv", 1.0)), float(layer.get("s_o", 1.0)),
               float(layer.get("s_gu", 1.0)), float(layer.get("s_d", 1.0)),
               layer["act_dtype"], int(layer.get("act_fp8", 0)), layer["kv_dtype"],
               float(layer.get("k_scale", 1.0)), float(layer.get("v_scale", 1.0)),
               (NORM if layer.get("norm") else 0) | (ROPE if layer.get("rope") else 0),
               float(layer.get("norm_eps", 1e-6)), float(layer.get("rope_base", 10000.0)))
    outs = {"qkv": np.empty((n, (nq + 2 * nkv) * d)), "attn": np.empty((n, nq * d)),
            "h": np.empty((n, D)), "y": np.empty((n, D))}
    if F > 0:
        outs["a"] = np.empty((n, F))
    if raw:  # each stored stage also before its rounding to the activation dtype
        outs["qkv_raw"] = np.empty_like(outs["qkv"])
        outs["attn_raw"] = np.empty_like(outs["attn"])
        if F > 0:
            outs["a_raw"] = np.empty_like(outs["a"])
    o = _Out(_ptr(outs["qkv"]), _ptr(outs["attn"]), _ptr(outs["h"]), _ptr(outs.get("a")),
             _ptr(outs["y"]), _ptr(outs.get("qkv_raw")), _ptr(outs.get("attn_raw")),
             _ptr(outs.get("a_raw")))
    h = hist.struct()
    rc = lib().orc_decode_step(ctypes.byref(L), ctypes.byref(h), n, _ptr(seq), _ptr(pos), _ptr(x),
                               ctypes.byref(o))
    if rc != 0:
        raise ValueError("oracle decode_step refused the rows (bad row or gap in a sequence)")
    del keep
    return outs
