#!/usr/bin/env python3
"""Benchmark of one decode step of a transformer layer over a paged KV pool.

Default workload: the bf16 7B-class batched decode layer (hidden 3584, 28 q /
4 kv heads, head_dim 128, FFN 18944, 768 rows, contexts 128 + U{1..128} with a
shared 2-page prompt prefix).  A step is one pass of the whole path: QKV
projection, append of each row's key/value, paged attention, output projection
+ residual, gate/up projection + SiLU, down projection + residual.

Prints one JSON line.  `value` = algorithmic HBM bytes of the step / measured
step time (GB/s), the step being decode_step captured once in a graph and
replayed (the eager time is reported beside it); the per-stage breakdown and
the dominant kernel's roofline are measured with HIP events on the stream the
kernels run on.  `configs` holds the same measurements for every workload
(tiny f32 layer, 0.6B layer at batch 1, 0.6B mixed batch of 512 decode rows
and a 256-row prompt chunk, the 7B batch-768 layer, the fp8 7B layer at batch
4,096); `cpu_baseline` times the fp64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
VALU_F32_PEAK_TFLOPS = 157.3
CONFIG_WORKLOADS = ["tiny-f32", "0.6b-b1-bf16", "0.6b-mixed-bf16", "7b-b768-prefix-bf16", "7b-b4096-fp8"]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed steps before each timed run: the card reaches its steady clock
    # after some 20-30 ms of back-to-back steps (a 7B batch-768 step replayed
    # from a graph: 492 us over the first 20 replays, 420-430 us from the 40th)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="7b-b768-prefix-bf16")
    ap.add_argument("--configs", default="all",
                    help="workloads measured besides the headline one: all, none, or a comma list")
    ap.add_argument("--sections", default="all",
                    help="parts to run: all, or a comma list of step, norm_rope, t1, t2, head, prefill, configs, cpu "
                         "(a profile of one part)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-t2", action="store_true", help="skip the small-batch GEMV pass")
    ap.add_argument("--no-head", action="store_true", help="skip the output-head (candidate rows) pass")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prompt-chunk (prefill) pass")
    ap.add_argument("--no-norm-rope", action="store_true", help="skip the step with norms and rotary positions")
    ap.add_argument("--cpu-max-s", type=float, default=150.0,
                    help="the oracle times a whole step when a 16-row pilot predicts at most this many seconds")
    ap.add_argument("--family", type=int, default=None, help="override the projection family")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy (known HBM bytes) for counter scaling")
    return ap.parse_args(argv)


def step_bytes(w, elem):
    """Algorithmic bytes and flops of one step, per stage: what the method
    must move, counted as the scope table's measurement rules state (a
    projection reads its weights once, its input rows in the activation dtype
    and writes its outputs, plus the residual read where there is one;
    attention reads the unique (physical page, valid slot) pairs once, shared
    pages once, plus q, out, table entries and row metadata; the append writes
    each row's key and value).  Passes an implementation adds (the bf16 cast
    of x, the bf16 copy of h, K-split partial sums) are not counted."""
    B, D, nq, nkv, d, F = w.n_rows, w.hidden, w.n_q, w.n_kv, w.head_dim, w.ffn
    sw, skv, sa = elem[w.w_dtype], elem[w.kv_dtype], elem[w.act_dtype]
    nqkv = (nq + 2 * nkv) * d
    fp8 = w.w_dtype == 2
    # unique (physical page, slot) pairs read by attention: slots < L of every row's pages
    seen = {}
    for r in range(B):
        s, L = int(w.seq[r]), int(w.pos[r]) + 1
        for lp in range((L + 31) // 32):
            pg = int(w.tables[s][lp])
            n = min(32, L - 32 * lp)
            seen[pg] = max(seen.get(pg, 0), n)
    kv_tokens = sum(seen.values())
    pages_touched = sum((int(p) + 32) // 32 for p in w.pos)
    # the fp8 tier quantises its projection inputs per row from the f32 (x, h)
    # or bf16 (attn, a) values: those are what it reads
    x_in = 4 if fp8 else sa
    st = {}
    st["qkv"] = nqkv * D * sw + B * D * x_in + B * nqkv * sa
    st["append"] = B * 2 * nkv * d * skv
    st["attention"] = kv_tokens * 2 * nkv * d * skv + B * nq * d * (sa + sa) + 4 * pages_touched + 8 * B
    st["wo"] = D * nq * d * sw + B * nq * d * sa + B * D * 4 * 2
    if F:
        st["gate_up"] = 2 * F * D * sw + B * D * x_in + B * F * sa
        st["down"] = D * F * sw + B * F * sa + B * D * 4 * 2
    flops = {"qkv": 2 * B * nqkv * D, "wo": 2 * B * D * nq * d}
    if F:
        flops["gate_up"] = 2 * B * 2 * F * D
        flops["down"] = 2 * B * D * F
    flops["attention"] = 4 * nq * d * int(sum(int(p) + 1 for p in w.pos))
    return st, flops, kv_tokens


def stage_peak(stage: str, family: int, w_dtype: int):
    """(bound, peak) of a stage's kernel: HBM for attention, the matrix-core
    peak of the operand type for the matrix-core families, the fp32 vector
    peak for the vector GEMV (whose small batches are HBM-bound anyway)."""
    if stage == "attention":
        return "hbm", None
    if family == 2:
        return "mfma", MFMA_PEAK_TFLOPS["fp8"]
    if family in (1, 3):
        return "mfma", MFMA_PEAK_TFLOPS["bf16"]
    return "alu", VALU_F32_PEAK_TFLOPS


def ideal_us(nbytes: float, flops: float, peak_tflops) -> float:
    """Time of a stage at its roofline: the larger of its bytes at the HBM
    peak and its flops at its compute peak."""
    t = nbytes / (HBM_PEAK_GBS * 1e9)
    if peak_tflops:
        t = max(t, flops / (peak_tflops * 1e12))
    return t * 1e6


# Sources of each stage's kernel: a counter summary is only valid for the code
# it was taken on.
def stage_sources(stage: str, family: int) -> list:
    if stage == "attention":
        return ["attention.hip"]
    return ["gemv.hip"] if family in (0, 3) else ["gemm.hip"]


def source_hash(stage: str, family: int) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_attn_amd", "csrc")
    for f in stage_sources(stage, family) + ["common.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _kv_file(path):
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def measured_traffic(stage: str, workload: str, family: int):
    """HBM bytes per launch of the stage's kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's
    reading for a copy of known size), or None if there is none or the kernel
    source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = _kv_file(path)
    if kv.get("source_sha256") != source_hash(stage, family):
        return None
    cb = float(kv["copy_bytes"])
    f = float(kv["fetch_kib_per_dispatch"]) * cb / float(kv["copy_fetch_kib"])
    w = float(kv["write_kib_per_dispatch"]) * cb / float(kv["copy_write_kib"])
    return int(round(f + w))


def traced_us(stage: str, workload: str, family: int):
    """Average duration of the stage's kernel(s) in the committed rocprofv3
    kernel trace of this workload's step (the stage alone, launched back to
    back, where the trace has it), or None if there is none or the kernel
    source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"step_{workload}.stages.txt")
    if not os.path.exists(path):
        return None
    kv = _kv_file(path)
    if kv.get(f"{stage}_source_sha256") != source_hash(stage, family):
        return None
    v = kv.get(f"{stage}_us_alone") or kv.get(f"{stage}_us_per_step")
    return float(v) if v else None


def copy_calibration():
    import torch
    n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written per copy
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 4 * n, "copies": 3}))


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def pct(ts):
    """median, p10, p90 of a list of times."""
    ts = sorted(ts)
    return ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Bench:
    def __init__(self, args):
        import torch
        self.args = args
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.gstream = torch.cuda.Stream()
        # cold runs: a 2 GiB buffer is read (a reduction, leaving no dirty
        # lines) before a timed call, so no pool page or weight is left in L2
        # or the 256 MB MALL
        self.flush = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
        self.flush_sum = torch.empty((), dtype=torch.float32, device="cuda")

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def cold(self):
        self.torch.sum(self.flush, 0, out=self.flush_sum)

    def timed(self, fn, reps, cold):
        """Median, p10, p90 (us) of `reps` calls, each between two events on the stream."""
        ts = []
        for _ in range(reps):
            if cold:
                self.cold()
            a, b = self.ev(), self.ev()
            a.record(self.stream)
            fn()
            b.record(self.stream)
            self.torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return pct(ts)

    def graph_steps(self, fn, steps, warmup):
        """fn captured once in a graph and replayed (us): the mean over `steps`
        replays back to back with an event before the first and after the
        last only (an event recorded between replays costs several us of its
        own), then the median, p10 and p90 of as many more replays, each
        between two events."""
        torch = self.torch
        gs = self.gstream
        gs.wait_stream(self.stream)
        with torch.cuda.stream(gs):
            fn(gs)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                fn(gs)
            for _ in range(warmup):
                g.replay()
            e0, e1 = self.ev(), self.ev()
            e0.record(gs)
            for _ in range(steps):
                g.replay()
            e1.record(gs)
            evs = [self.ev() for _ in range(steps + 1)]
            evs[0].record(gs)
            for i in range(steps):
                g.replay()
                evs[i + 1].record(gs)
        torch.cuda.synchronize()
        ts = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps)]
        mean = e0.elapsed_time(e1) * 1e3 / steps
        med, p10, p90 = pct(ts)
        del g
        return med, p10, p90, mean

    # ------------------------------------------------------------ one workload
    def measure(self, w, detail: bool):
        """Step and per-stage timings of workload w.  detail: also keeps the
        objects the headline's extra passes need."""
        import numpy as np
        import paged_kv_decode_attn_amd as pkd
        import gpu_harness as H
        torch = self.torch
        args = self.args
        pool = H.GpuPool(w)
        layer = H.GpuLayer(w, batch_hint=w.n_rows)  # engine built for this batch: fixed K splits
        L = layer.layer
        B, D, nq, nkv, d, F = w.n_rows, w.hidden, w.n_q, w.n_kv, w.head_dim, w.ffn
        stream = self.stream
        s_t, p_t = H.rows_tensors(w.seq, w.pos)
        distinct = len(set(w.seq.tolist())) == B  # pure decode batch: the append runs inside attention
        rows = pkd.make_rows(s_t, p_t, distinct)
        x = w.x.cuda().contiguous()
        y = torch.empty((B, D), dtype=torch.float32, device="cuda")
        ws = H.aligned_empty(pkd.pkd_step_workspace_bytes(L, pool.handle, B))
        for _ in range(args.warmup):
            pkd.decode_step(L, pool.handle, rows, x, y, ws)
        torch.cuda.synchronize()
        e0, e1 = self.ev(), self.ev()
        e0.record(stream)
        for _ in range(args.steps):
            pkd.decode_step(L, pool.handle, rows, x, y, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) / args.steps * 1e3
        pkd.pkd_pool_check(pool.handle)
        med, p10, p90, mean = self.graph_steps(
            lambda st: pkd.decode_step(L, pool.handle, rows, x, y, ws, stream=st), args.steps, args.warmup)
        pkd.pkd_pool_check(pool.handle)
        # cold: each eager step after a flush of L2 and the MALL
        c_med, c_p10, c_p90 = self.timed(lambda: pkd.decode_step(L, pool.handle, rows, x, y, ws),
                                         max(args.steps, 10), True)
        log(f"{w.name}: decode_step graph replay {mean:.1f} us (median {med:.1f}), eager {us_eager:.1f}, "
            f"cold {c_med:.1f}")

        # ---- per stage: the same kernels, launched stage by stage through the
        # public entry points, with events between the stages on the stream
        act = w.act_dtype
        fp8 = w.w_dtype == 2
        ebytes = {0: 4, 1: 2, 2: 1}
        nqkv = (nq + 2 * nkv) * d
        tdt = torch.float32 if act == 0 else torch.int16
        qkv = torch.empty((B, nqkv), dtype=tdt, device="cuda")
        att = torch.empty((B, nq * d), dtype=tdt, device="cuda")
        h = torch.empty((B, D), dtype=torch.float32, device="cuda")
        hb = torch.empty((B, D), dtype=torch.int16, device="cuda")
        xb = x.to(torch.bfloat16).view(torch.int16)
        a_ = torch.empty((B, max(F, 1)), dtype=tdt, device="cuda")
        mats = [L.w_qkv, L.w_o] + ([L.w_gate_up, L.w_down] if F else [])
        pws = max(pkd.pkd_gemv_workspace_bytes(m, B) for m in mats)
        pws = H.aligned_empty(pws) if pws else None
        aws = H.aligned_empty(pkd.pkd_attn_workspace_bytes(pool.handle, nq, B))

        def st_qkv():
            xin, xdt = (x, 0) if (fp8 or act == 0) else (xb, 1)
            pkd.gemv_rows(L.w_qkv, xin, xdt, B, qkv, act, ws=pws)

        def st_attn():
            pkd.paged_attn_decode(pool.handle, rows, nq, q_c, k_c, v_c, att, act, aws)

        def st_wo():
            pkd.gemv_rows(L.w_o, att, act, B, h, 0, residual=x, y_bf16=(None if (fp8 or act == 0) else hb), ws=pws)

        def st_gu():
            hin, hdt = (h, 0) if (fp8 or act == 0) else (hb, 1)
            pkd.gemv_rows(L.w_gate_up, hin, hdt, B, a_, act, silu_pair=True, ws=pws)

        def st_down():
            pkd.gemv_rows(L.w_down, a_, act, B, y, 0, residual=h, ws=pws)

        st_qkv()
        torch.cuda.synchronize()
        q3 = qkv.view(B, nq + 2 * nkv, d)
        q_c = q3[:, :nq].contiguous()
        k_c = q3[:, nq:nq + nkv].contiguous()
        v_c = q3[:, nq + nkv:].contiguous()
        stages = [("qkv", st_qkv), ("attention", st_attn), ("wo", st_wo)]
        if F:
            stages += [("gate_up", st_gu), ("down", st_down)]
        for _ in range(args.warmup):
            for _, f in stages:
                f()
        torch.cuda.synchronize()
        evs = [[self.ev() for _ in range(len(stages) + 1)] for _ in range(args.steps)]
        for k in range(args.steps):
            evs[k][0].record(stream)
            for i, (_, f) in enumerate(stages):
                f()
                evs[k][i + 1].record(stream)
        torch.cuda.synchronize()
        stage_us = {}
        for i, (name, _) in enumerate(stages):
            stage_us[name] = float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)])) * 1e3
        pkd.pkd_pool_check(pool.handle)
        sbytes, sflops, kv_tokens = step_bytes(w, ebytes)
        sbytes_m = dict(sbytes)
        sbytes_m["attention"] = sbytes["attention"] + sbytes.pop("append")
        total_bytes = sum(sbytes_m.values())
        total_flops = sum(sflops.values())
        fams = {"qkv": L.w_qkv.family, "wo": L.w_o.family, "gate_up": L.w_gate_up.family,
                "down": L.w_down.family, "attention": -1}
        kernels, ideal_total = {}, 0.0
        for name, us in stage_us.items():
            kb, fl = sbytes_m[name], sflops.get(name, 0)
            bound, peak = stage_peak(name, int(fams[name]), w.w_dtype)
            ideal = ideal_us(kb, fl, peak)
            ideal_total += ideal
            kernels[name] = {"us": round(us, 2), "bytes": int(kb), "GB_s": round(kb / us / 1e3, 1),
                             "hbm_frac": round(kb / us / 1e3 / HBM_PEAK_GBS, 4),
                             "TFLOP_s": round(fl / us / 1e6, 1) if fl else None,
                             "bound": bound, "ideal_us": round(ideal, 2), "roofline_frac": round(ideal / us, 4)}
        dom = max(stage_us, key=stage_us.get)
        # the dominant stage alone, launched back to back between two events:
        # its kernels' average duration without an event pair around each launch
        dom_fn = dict(stages)[dom]
        e0.record(stream)
        for _ in range(args.steps):
            dom_fn()
        e1.record(stream)
        torch.cuda.synchronize()
        dom_us = e0.elapsed_time(e1) / args.steps * 1e3
        pkd.pkd_pool_check(pool.handle)
        bound, peak = stage_peak(dom, int(fams[dom]), w.w_dtype)
        if bound == "hbm" or (bound == "alu" and sbytes_m[dom] / (HBM_PEAK_GBS * 1e9) >=
                              sflops.get(dom, 0) / (peak * 1e12)):
            bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
            achieved = sbytes_m[dom] / dom_us / 1e3
        else:
            unit = "TFLOP/s"
            achieved = sflops[dom] / dom_us / 1e6
        fam = int(fams[dom]) if dom != "attention" else 0
        tr_us = traced_us(dom, w.name, fam)
        roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                    "frac": round(achieved / peak, 4), "traffic": measured_traffic(dom, w.name, fam),
                    "algorithmic_bytes": int(sbytes_m[dom]), "us": round(dom_us, 2),
                    "us_between_stages": round(stage_us[dom], 2), "trace_us": tr_us}
        rec = {"rows": B, "dtype": {0: "f32", 1: "bf16", 2: "fp8"}[w.w_dtype], "projection_family": int(L.w_qkv.family),
               "us_per_step": round(mean, 2), "median_us": round(med, 2), "p10_us": round(p10, 2),
               "p90_us": round(p90, 2), "us_per_step_eager": round(us_eager, 2),
               "cold": {"us": round(c_med, 2), "p10_us": round(c_p10, 2), "p90_us": round(c_p90, 2)},
               "step_bytes": int(total_bytes), "step_flops": int(total_flops),
               "GB_s": round(total_bytes / mean / 1e3, 1), "hbm_frac": round(total_bytes / mean / 1e3 / HBM_PEAK_GBS, 4),
               "ideal_us": round(ideal_total, 2), "roofline_frac": round(ideal_total / mean, 4),
               "kv_tokens_unique": int(kv_tokens), "kernels": kernels, "dominant": roofline}
        ctx = None
        if detail:
            ctx = dict(pool=pool, layer=layer, rows=rows, x=x, y=y, ws=ws, st_attn=st_attn,
                       attn_bytes=sbytes_m["attention"], total_bytes=total_bytes)
        return rec, ctx

    # ------------------------------------------------------------ headline extras
    def norm_rope_step(self, w, ctx):
        import paged_kv_decode_attn_amd as pkd
        import gpu_harness as H
        L = ctx["layer"].layer
        Ln = pkd.pkd_layer.from_buffer_copy(L)
        Ln.flags, Ln.norm_eps, Ln.rope_base = pkd.LAYER_NORM | pkd.LAYER_ROPE, 1e-6, 10000.0
        pool, rows, x, y = ctx["pool"], ctx["rows"], ctx["x"], ctx["y"]
        wsn = H.aligned_empty(pkd.pkd_step_workspace_bytes(Ln, pool.handle, w.n_rows))
        med, p10, p90, mean = self.graph_steps(
            lambda st: pkd.decode_step(Ln, pool.handle, rows, x, y, wsn, stream=st), self.args.steps,
            self.args.warmup)
        pkd.pkd_pool_check(pool.handle)
        log(f"decode_step with norm + rope, graph replay {mean:.1f} us")
        return {"us_per_step": round(mean, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2)}

    def t1(self, ctx):
        ab = ctx["attn_bytes"]
        res = {"bytes": int(ab)}
        for mode in ("cold", "warm"):
            med, p10, p90 = self.timed(ctx["st_attn"], max(self.args.steps, 10), mode == "cold")
            res[mode] = {"us": round(med, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2),
                         "GB_s": round(ab / med / 1e3, 1), "hbm_frac": round(ab / med / 1e3 / HBM_PEAK_GBS, 4)}
        return res

    def t2(self, w):
        """The GEMV over every weight matrix of the layer at decode batches 1..16, cold."""
        import paged_kv_decode_attn_amd as pkd
        import gpu_harness as H
        torch = self.torch
        B, D, nq, nkv, d, F = w.n_rows, w.hidden, w.n_q, w.n_kv, w.head_dim, w.ffn
        nqkv = (nq + 2 * nkv) * d
        res = {"matrices": "W_qkv, W_o, [W_gate; W_up], W_down", "family": 0}
        wbytes = 2 * (nqkv * D + D * nq * d + 2 * F * D + D * F)
        for t2_fam in (0, 3):
            g_obj = H.GpuLayer(w, family=t2_fam)  # same weights; the object owns the device copies
            g_layer = g_obj.layer
            dest = res if t2_fam == 0 else res.setdefault("family3_matrix_core_gemv", {})
            for nb in (1, 4, 8, 16):
                xs = (torch.randn((nb, max(D, F, nq * d)), device="cuda") * 0.5).to(torch.bfloat16).view(torch.int16)
                oq = torch.empty((nb, nqkv), dtype=torch.int16, device="cuda")
                oh = torch.empty((nb, D), dtype=torch.float32, device="cuda")
                og = torch.empty((nb, F), dtype=torch.int16, device="cuda")
                res_in = torch.zeros((nb, D), dtype=torch.float32, device="cuda")
                xd, xa, xf = xs[:, :D].contiguous(), xs[:, :nq * d].contiguous(), xs[:, :F].contiguous()
                per = {}

                def one(name):
                    if name == "qkv":
                        pkd.gemv_rows(g_layer.w_qkv, xd, 1, nb, oq, 1)
                    elif name == "wo":
                        pkd.gemv_rows(g_layer.w_o, xa, 1, nb, oh, 0, residual=res_in)
                    elif name == "gate_up":
                        pkd.gemv_rows(g_layer.w_gate_up, xd, 1, nb, og, 1, silu_pair=True)
                    else:
                        pkd.gemv_rows(g_layer.w_down, xf, 1, nb, oh, 0, residual=res_in)

                def gemv_pass():
                    for name in ("qkv", "wo", "gate_up", "down"):
                        one(name)
                for _ in range(3):
                    gemv_pass()
                med, p10, p90 = self.timed(gemv_pass, max(self.args.steps, 10), True)
                byt = wbytes + nb * 2 * (D + nq * d + D + F) + nb * (2 * nqkv + 8 * D + 2 * F + 8 * D)
                ent = {"us": round(med, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2), "bytes": int(byt),
                       "GB_s": round(byt / med / 1e3, 1), "hbm_frac": round(byt / med / 1e3 / HBM_PEAK_GBS, 4)}
                if nb == 1:
                    # each matrix alone, cold: its streaming rate
                    mb = {"qkv": 2 * nqkv * D, "wo": 2 * D * nq * d, "gate_up": 4 * F * D, "down": 2 * D * F}
                    for name in ("qkv", "wo", "gate_up", "down"):
                        m_med, _, _ = self.timed(lambda: one(name), max(self.args.steps, 10), True)
                        per[name] = {"us": round(m_med, 2), "GB_s": round(mb[name] / m_med / 1e3, 1),
                                     "hbm_frac": round(mb[name] / m_med / 1e3 / HBM_PEAK_GBS, 4)}
                    ent["per_matrix"] = per
                dest[f"B{nb}"] = ent
            del g_obj
        return res

    def head(self):
        """Output head over a tied embedding (151,936 x 2,048 bf16, 593.5 MiB):
        the dense head at batch 1 against the candidate-row head, whose rows
        carry trie-shaped lists of 1..28 candidates, cold."""
        import paged_kv_decode_attn_amd as pkd
        import workloads as wl
        torch = self.torch
        V, HD, HC = wl.HEAD_VOCAB, wl.HEAD_HIDDEN, wl.HEAD_MAX_CAND
        gh = torch.Generator(device="cuda").manual_seed(7)
        Wh = torch.empty((V, HD), dtype=torch.int16, device="cuda")
        for i in range(0, V, 16384):
            blk = torch.randn((min(16384, V - i), HD), generator=gh, device="cuda") * 0.02
            Wh[i:i + blk.shape[0]] = blk.to(torch.bfloat16).view(torch.int16)
        Mh = pkd.make_matrix(Wh, V, HD, 1, 1.0, 0)
        res = {"vocab": V, "hidden": HD, "max_cand": HC, "dtype": "bf16", "matrix_bytes": V * HD * 2}
        reps = max(self.args.steps, 10)
        for nb in (1, 64, 512):
            xh = (torch.randn((nb, HD), generator=gh, device="cuda")).to(torch.bfloat16).view(torch.int16)
            cand, n_cand = wl.head_candidates(nb, V, HC, 1000 + nb)
            cd, nd = torch.from_numpy(cand).cuda(), torch.from_numpy(n_cand).cuda()
            yh = torch.empty((nb, HC), device="cuda")
            gbytes = int(n_cand.sum()) * HD * 2 + nb * HD * 2 + int(n_cand.sum()) * 4 + nb * HC * 4 + nb * 4
            for _ in range(3):
                pkd.gemv_gather_rows(Mh, xh, 1, nb, cd, nd, HC, yh)
            med, p10, p90 = self.timed(lambda: pkd.gemv_gather_rows(Mh, xh, 1, nb, cd, nd, HC, yh), reps, True)
            ent = {"gathered_us": round(med, 2), "gathered_p10_us": round(p10, 2), "gathered_p90_us": round(p90, 2),
                   "gathered_bytes": gbytes, "gathered_GB_s": round(gbytes / med / 1e3, 1),
                   "mean_candidates": round(float(n_cand.mean()), 2)}
            if nb == 1:
                yd = torch.empty((nb, V), device="cuda")
                for _ in range(3):
                    pkd.gemv_rows(Mh, xh, 1, nb, yd, 0)
                dmed, _, _ = self.timed(lambda: pkd.gemv_rows(Mh, xh, 1, nb, yd, 0), reps, True)
                dbytes = V * HD * 2 + HD * 2 + V * 4
                ent.update({"dense_us": round(dmed, 2), "dense_bytes": dbytes,
                            "dense_GB_s": round(dbytes / dmed / 1e3, 1),
                            "dense_hbm_frac": round(dbytes / dmed / 1e3 / HBM_PEAK_GBS, 4),
                            "speedup_vs_dense": round(dmed / med, 1)})
                del yd
            res[f"B{nb}"] = ent
        del Wh, Mh
        return res

    def prefill(self, w):
        """Prefill of one 2,662-token prompt in 256-token chunks through the same
        layer shape: the chunk as one step (matrix-core projections, shared-tile
        attention) against the same 256 tokens one step each (vector GEMV at
        batch 1), and the chunk's attention with shared tiles against per-row
        (both replayed from graphs)."""
        import paged_kv_decode_attn_amd as pkd
        import workloads as wl
        import gpu_harness as H
        torch = self.torch
        D, nq, d = w.hidden, w.n_q, w.head_dim
        lname = "7b" if D == 3584 else "0.6b"
        res = {"layer": lname, "prompt_tokens": 2662, "chunk_tokens": 256, "attn_chunk_pages": 8}
        for p0 in (1024, 2304):
            wp = wl.make("prefill-chunk", "cuda", layer=lname, p0=p0, n=256, seed=3)
            poolp = H.GpuPool(wp)
            layp = H.GpuLayer(wp, batch_hint=256)
            nP = wp.n_rows
            sp, pp = H.rows_tensors(wp.seq, wp.pos)
            rows_p = pkd.make_rows(sp, pp, False)
            xp = wp.x.contiguous()
            yp = torch.empty((nP, D), dtype=torch.float32, device="cuda")
            wsp = H.aligned_empty(pkd.pkd_step_workspace_bytes(layp.layer, poolp.handle, nP))
            _, _, _, us_chunk = self.graph_steps(
                lambda st: pkd.decode_step(layp.layer, poolp.handle, rows_p, xp, yp, wsp, stream=st),
                self.args.steps, self.args.warmup)
            pkd.pkd_pool_check(poolp.handle)
            lay1 = H.GpuLayer(wp, family=0)
            ws1 = H.aligned_empty(pkd.pkd_step_workspace_bytes(lay1.layer, poolp.handle, 1))
            y1 = torch.empty((1, D), dtype=torch.float32, device="cuda")
            one_rows = [pkd.make_rows(sp[i:i + 1], pp[i:i + 1], True) for i in range(nP)]
            xs1 = [xp[i:i + 1] for i in range(nP)]

            def token_by_token():
                for i in range(nP):
                    pkd.decode_step(lay1.layer, poolp.handle, one_rows[i], xs1[i], y1, ws1)
            token_by_token()
            torch.cuda.synchronize()
            e0, e1 = self.ev(), self.ev()
            e0.record(self.stream)
            token_by_token()
            e1.record(self.stream)
            torch.cuda.synchronize()
            us_tokens = e0.elapsed_time(e1) * 1e3
            qa = (torch.randn((nP, nq, d), device="cuda")).to(torch.bfloat16).view(torch.int16)
            oa = torch.empty((nP, nq, d), dtype=torch.int16, device="cuda")
            wsa = H.aligned_empty(pkd.pkd_attn_workspace_bytes(poolp.handle, nq, nP))
            rows_row = pkd.make_rows(sp, pp, True)  # no append: the per-row kernels, tiles off
            # the chunk's attention alone, replayed from a graph like the step (no host launch gaps)
            reps = max(self.args.steps, 10)
            att_t, _, _, _ = self.graph_steps(
                lambda st: pkd.paged_attn_decode(poolp.handle, rows_p, nq, qa, None, None, oa, 1, wsa, stream=st),
                reps, 3)
            att_r, _, _, _ = self.graph_steps(
                lambda st: pkd.paged_attn_decode(poolp.handle, rows_row, nq, qa, None, None, oa, 1, wsa, stream=st),
                reps, 3)
            # causal attention flops of the chunk: q.K and P.V over each row's context
            att_flops = sum(4 * nq * d * (int(p) + 1) for p in wp.pos)
            res[f"pos{p0}"] = {
                "us_chunk_step": round(us_chunk, 1), "tokens_per_s": round(nP / us_chunk * 1e6),
                "us_token_by_token": round(us_tokens, 1), "speedup_vs_token_by_token": round(us_tokens / us_chunk, 1),
                "attention_us_shared_tiles": round(att_t, 2), "attention_us_per_row": round(att_r, 2),
                "attention_gflop": round(att_flops / 1e9, 3),
                "attention_tflops_shared_tiles": round(att_flops / att_t / 1e6, 1),
                "attention_mfma_frac_shared_tiles": round(att_flops / att_t / 1e6 / MFMA_PEAK_TFLOPS["bf16"], 4)}
            del wp, poolp, layp, lay1
        return res


def cpu_baseline(w, total_bytes, max_s):
    """The fp64 oracle (as it stands) on the host cores: a whole step of the
    workload when a 16-row pilot predicts at most max_s seconds, else the
    time per row of a 64-row sample scaled to the batch."""
    import numpy as np
    import workloads as wl
    from oracle import oracle as orc
    B = w.n_rows
    lay = wl.layer_dict(w)

    def run(nr):
        rws = np.arange(nr)
        seqs = np.unique(w.seq[rws])
        hk, hv = wl.history_lists(w, seqs)
        hist = orc.History(hk, hv, w.kv_dtype, w.n_kv, w.head_dim)
        xs = w.x[:nr].cpu().numpy()
        t0 = time.perf_counter()
        orc.decode_step(lay, hist, w.seq[rws], w.pos[rws], xs)
        return time.perf_counter() - t0
    pilot_rows = min(16, B)
    pilot = run(pilot_rows)
    predicted = pilot / pilot_rows * B
    if predicted <= max_s:
        log(f"cpu baseline: oracle on the whole step ({B} rows, predicted {predicted:.0f} s, {orc.threads()} threads)")
        t = run(B)
        per_step, sample = t, f"fp64 oracle, whole decode step of all {B} rows ({t:.1f} s)"
    else:
        nr = min(64, B)
        log(f"cpu baseline: oracle on {nr} of {B} rows (a whole step predicted at {predicted:.0f} s)")
        t = run(nr)
        per_step = t / nr * B
        sample = f"fp64 oracle decode step of the first {nr} of {B} rows ({t:.1f} s), time per row x {B} rows"
    return {"value": round(total_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": orc.threads(),
            "kind": "oracle", "us_per_step": round(per_step * 1e6, 1), "sample": sample, "cpu_model": cpu_model()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path is a single-GPU kernel set with no "
              f"collective leg (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import workloads as wl

    allp = {"step", "norm_rope", "t1", "t2", "head", "prefill", "configs", "cpu"}
    sec = allp if args.sections == "all" else set(args.sections.split(","))
    if sec - allp:
        print(f"unknown sections {sorted(sec - allp)}", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    bench = Bench(args)
    for flag, part in (("no_norm_rope", "norm_rope"), ("no_t2", "t2"), ("no_head", "head"),
                       ("no_prefill", "prefill"), ("no_cpu_baseline", "cpu")):
        if getattr(args, flag):
            sec.discard(part)
    if args.configs == "none":
        sec.discard("configs")
    kw = {} if args.family is None else {"family": args.family}
    log(f"generating workload {args.workload}")
    w = wl.make(args.workload, "cuda", **kw)
    rec = ctx = nr = t1 = None
    total_bytes = None
    if sec & {"step", "norm_rope", "t1", "cpu"}:
        rec, ctx = bench.measure(w, detail=True)
        total_bytes = ctx["total_bytes"]
        nr = bench.norm_rope_step(w, ctx) if "norm_rope" in sec else None
        t1 = bench.t1(ctx) if "t1" in sec else None
        del ctx
    t2 = bench.t2(w) if ("t2" in sec and w.ffn and w.w_dtype == 1) else None
    head = bench.head() if "head" in sec else None
    pre = bench.prefill(w) if ("prefill" in sec and w.w_dtype == 1 and w.ffn) else None
    if rec is None:  # a profile of one part: no step line
        print(json.dumps({"t2_gemv": t2, "output_head": head, "prefill": pre}))
        return
    configs = {w.name: {k: v for k, v in rec.items() if k not in ("kernels",)}}
    names = [] if "configs" not in sec else (
        CONFIG_WORKLOADS if args.configs == "all" else args.configs.split(","))
    for name in names:
        if name == w.name:
            continue
        log(f"generating workload {name}")
        wc = wl.make(name, "cuda")
        rc, _ = bench.measure(wc, detail=False)
        configs[name] = rc
        del wc
        torch.cuda.empty_cache()
    cpu = cpu_baseline(w, total_bytes, args.cpu_max_s) if "cpu" in sec else None
    line = {
        "metric": "decode-step us and achieved HBM GB/s (% of peak), paged attn + GEMV",
        "value": rec["GB_s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(rec["us_per_step"] / 1e3, 4), "us_per_step": rec["us_per_step"],
        "p10_us": rec["p10_us"], "p90_us": rec["p90_us"], "us_per_step_eager": rec["us_per_step_eager"],
        "us_per_step_cold": rec["cold"]["us"],
        "hbm_frac": rec["hbm_frac"], "roofline_frac_step": rec["roofline_frac"], "ideal_us": rec["ideal_us"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": rec["dtype"], "data": "synthetic",
        "config": {"workload": w.name, "rows": w.n_rows, "hidden": w.hidden, "q_heads": w.n_q, "kv_heads": w.n_kv,
                   "head_dim": w.head_dim, "ffn": w.ffn, "page_tokens": 32, "kv_tokens_unique": rec["kv_tokens_unique"],
                   "projection_family": rec["projection_family"], "parallelism": "none (1 GPU)"},
        "step_bytes": rec["step_bytes"],
        "kernels": rec["kernels"],
        "roofline": rec["dominant"],
        "norm_rope_step": nr,
        "t1_attention": t1,
        "t2_gemv": t2,
        "output_head": head,
        "prefill": pre,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
