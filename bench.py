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
kernels run on.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="7b-b768-prefix-bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-t2", action="store_true", help="skip the small-batch GEMV pass")
    ap.add_argument("--no-head", action="store_true", help="skip the output-head (candidate rows) pass")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prompt-chunk (prefill) pass")
    ap.add_argument("--cpu-rows", type=int, default=128)
    ap.add_argument("--family", type=int, default=None, help="override the projection family")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy (known HBM bytes) for counter scaling")
    return ap.parse_args()


def step_bytes(w, elem):
    """Algorithmic bytes of one step, per stage (what the method must move)."""
    import numpy as np
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
    xin = 1 if fp8 else sa  # projection input bytes per element (fp8 codes or act dtype)
    st = {}
    st["cast"] = 0 if fp8 or w.act_dtype == 0 else B * D * (4 + 2)
    st["qkv"] = nqkv * D * sw + B * D * (4 if fp8 else xin) + B * nqkv * sa
    st["append"] = B * 2 * nkv * d * skv + B * 2 * nkv * d * sa
    st["attention"] = (kv_tokens * 2 * nkv * d * skv + B * nq * d * (sa + sa) + 4 * pages_touched + 8 * B)
    st["wo"] = D * nq * d * sw + B * nq * d * sa + B * D * 4 * 2 + (0 if fp8 else B * D * 2)
    if F:
        st["gate_up"] = 2 * F * D * sw + B * D * (4 if fp8 else 2) + B * F * sa
        st["down"] = D * F * sw + B * F * sa + B * D * 4 * 2
    flops = {"qkv": 2 * B * nqkv * D, "wo": 2 * B * D * nq * d}
    if F:
        flops["gate_up"] = 2 * B * 2 * F * D
        flops["down"] = 2 * B * D * F
    flops["attention"] = 4 * nq * d * int(sum(int(p) + 1 for p in w.pos))
    return st, flops, kv_tokens


# Sources of each stage's kernel: a counter summary is only valid for the code
# it was taken on.
def stage_sources(stage: str, family: int) -> list:
    if stage == "attention":
        return ["attention.hip"]
    return ["gemv.hip"] if family == 0 else ["gemm.hip"]


def source_hash(stage: str, family: int) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_attn_amd", "csrc")
    for f in stage_sources(stage, family) + ["common.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(stage: str, workload: str, family: int):
    """HBM bytes per launch of the stage's kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's
    reading for a copy of known size), or None if there is none or the kernel
    source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash(stage, family):
        return None
    cb = float(kv["copy_bytes"])
    f = float(kv["fetch_kib_per_dispatch"]) * cb / float(kv["copy_fetch_kib"])
    w = float(kv["write_kib_per_dispatch"]) * cb / float(kv["copy_write_kib"])
    return int(round(f + w))


def copy_calibration():
    import torch
    n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written per copy
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 4 * n, "copies": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path is a single-GPU kernel set with no "
              f"collective leg (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import numpy as np
    import torch

    import paged_kv_decode_attn_amd as pkd
    import workloads as wl
    import gpu_harness as H

    torch.cuda.set_device(0)
    kw = {} if args.family is None else {"family": args.family}
    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    w = wl.make(args.workload, "cuda", **kw)
    pool = H.GpuPool(w)
    layer = H.GpuLayer(w, batch_hint=w.n_rows)  # engine built for this batch: fixed K splits
    L = layer.layer
    B, D, nq, nkv, d, F = w.n_rows, w.hidden, w.n_q, w.n_kv, w.head_dim, w.ffn
    stream = torch.cuda.current_stream()
    s_t, p_t = H.rows_tensors(w.seq, w.pos)
    distinct = len(set(w.seq.tolist())) == B  # pure decode batch: the append runs inside attention
    rows = pkd.make_rows(s_t, p_t, distinct)
    x = w.x.contiguous()
    y = torch.empty((B, D), dtype=torch.float32, device="cuda")
    ws = H.aligned_empty(pkd.pkd_step_workspace_bytes(L, pool.handle, B))

    # ---------------------------------------------------------------- whole step
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        pkd.decode_step(L, pool.handle, rows, x, y, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        pkd.decode_step(L, pool.handle, rows, x, y, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / args.steps
    pkd.pkd_pool_check(pool.handle)
    print(f"[bench] decode_step eager {ms_eager * 1e3:.1f} us", file=sys.stderr, flush=True)

    # The same step captured once in a graph and replayed, as a serving loop
    # runs it (identical kernels and arguments; only the per-launch host and
    # queue gaps go).
    gstream = torch.cuda.Stream()
    gstream.wait_stream(stream)
    with torch.cuda.stream(gstream):
        pkd.decode_step(L, pool.handle, rows, x, y, ws, stream=gstream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gstream):
            pkd.decode_step(L, pool.handle, rows, x, y, ws, stream=gstream)
        for _ in range(args.warmup):
            graph.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(gstream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(gstream)
    torch.cuda.synchronize()
    ms_step = g0.elapsed_time(g1) / args.steps
    pkd.pkd_pool_check(pool.handle)
    print(f"[bench] decode_step graph replay {ms_step * 1e3:.1f} us", file=sys.stderr, flush=True)

    # The same step with both RMSNorms folded into the projections and rotary
    # positions on q and k (same weights, standing for gain-folded ones).
    Ln = pkd.pkd_layer.from_buffer_copy(L)
    Ln.flags, Ln.norm_eps, Ln.rope_base = pkd.LAYER_NORM | pkd.LAYER_ROPE, 1e-6, 10000.0
    wsn = H.aligned_empty(pkd.pkd_step_workspace_bytes(Ln, pool.handle, B))
    with torch.cuda.stream(gstream):
        pkd.decode_step(Ln, pool.handle, rows, x, y, wsn, stream=gstream)
        graph_n = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_n, stream=gstream):
            pkd.decode_step(Ln, pool.handle, rows, x, y, wsn, stream=gstream)
        for _ in range(args.warmup):
            graph_n.replay()
        g0.record(gstream)
        for _ in range(args.steps):
            graph_n.replay()
        g1.record(gstream)
    torch.cuda.synchronize()
    ms_step_nr = g0.elapsed_time(g1) / args.steps
    pkd.pkd_pool_check(pool.handle)
    print(f"[bench] decode_step with norm + rope, graph replay {ms_step_nr * 1e3:.1f} us", file=sys.stderr,
          flush=True)

    # ---------------------------------------------------------------- per stage
    # The same kernels with the same shapes, launched stage by stage through the
    # public entry points, with events between stages on the same stream.
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
    pws = max(pkd.pkd_gemv_workspace_bytes(m, B) for m in (L.w_qkv, L.w_o, L.w_gate_up, L.w_down))
    pws = H.aligned_empty(pws) if pws else None
    aws = H.aligned_empty(pkd.pkd_attn_workspace_bytes(pool.handle, nq, B))
    es = ebytes[act]
    stages = []

    def st_qkv():
        xin, xdt = (x, 0) if (fp8 or act == 0) else (xb, 1)
        pkd.gemv_rows(L.w_qkv, xin, xdt, B, qkv, act, ws=pws)

    def st_append_attn():
        # q, k_new, v_new as separate contiguous tensors (paged_attn_decode takes dense rows)
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
    stages = [("qkv", st_qkv), ("attention", st_append_attn), ("wo", st_wo)]
    if F:
        stages += [("gate_up", st_gu), ("down", st_down)]
    for _ in range(args.warmup):
        for _, f in stages:
            f()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        evs[k][0].record(stream)
        for i, (_, f) in enumerate(stages):
            f()
            evs[k][i + 1].record(stream)
    torch.cuda.synchronize()
    stage_us = {}
    for i, (name, _) in enumerate(stages):
        stage_us[name] = float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)])) * 1e3
    sbytes, sflops, kv_tokens = step_bytes(w, ebytes)
    sbytes_m = dict(sbytes)
    sbytes_m["attention"] = sbytes["attention"] + sbytes["append"]
    total_bytes = sum(sbytes.values())
    kernels = {}
    for name, us in stage_us.items():
        kb = sbytes_m.get(name, 0)
        fl = sflops.get(name, 0)
        kernels[name] = {"us": round(us, 2), "bytes": int(kb), "GB_s": round(kb / us / 1e3, 1),
                         "hbm_frac": round(kb / us / 1e3 / HBM_PEAK_GBS, 4),
                         "TFLOP_s": round(fl / us / 1e6, 1) if fl else None}
    # dominant kernel: longest stage
    dom = max(stage_us, key=stage_us.get)
    dt = "fp8" if fp8 else "bf16"
    fam = L.w_gate_up.family if F else L.w_qkv.family
    if dom == "attention" or fam == 0:
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
        achieved = sbytes_m[dom] / stage_us[dom] / 1e3
    else:
        bound, unit = "mfma", "TFLOP/s"
        peak = MFMA_PEAK_TFLOPS["bf16"] if (fam == 1 or not fp8) else MFMA_PEAK_TFLOPS["fp8"]
        achieved = sflops[dom] / stage_us[dom] / 1e6
    roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(dom, w.name, int(fam)),
                "algorithmic_bytes": int(sbytes_m[dom])}
    value = total_bytes / (ms_step * 1e-3) / 1e9

    # ---------------------------------------------------------------- attention and GEMV alone
    # t1_attention: append + paged attention alone on this workload's pool and rows, cold
    # (a 2 GiB buffer is read before every rep, outside the events, so no page
    # is left in L2 or the 256 MB MALL; read, not written, so that no dirty
    # lines are left to be written back during the timed call) and warm.
    # t2_gemv: the vector-family GEMV over every weight matrix of the layer at
    # decode batches 1..16, cold.
    flush = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    flush_sum = torch.empty((), dtype=torch.float32, device="cuda")

    def timed(fn, reps, cold):
        ts = []
        for _ in range(reps):
            if cold:
                torch.sum(flush, 0, out=flush_sum)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        ts.sort()
        return ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]

    ab = sbytes_m["attention"]
    t1_res = {"bytes": int(ab)}
    for mode in ("cold", "warm"):
        med, p10, p90 = timed(st_append_attn, max(args.steps, 10), mode == "cold")
        t1_res[mode] = {"us": round(med, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2),
                    "GB_s": round(ab / med / 1e3, 1), "hbm_frac": round(ab / med / 1e3 / HBM_PEAK_GBS, 4)}
    t2_res = None
    if not args.no_t2 and F and w.w_dtype == 1:
        t2_res = {"matrices": "W_qkv, W_o, [W_gate; W_up], W_down", "family": 0}
        wbytes = 2 * (nqkv * D + D * nq * d + 2 * F * D + D * F)
        # the vector family (the graded one), then the same pass on the matrix-core GEMV family
        for t2_fam in (0, 3):
            g_obj = H.GpuLayer(w, family=t2_fam)  # same weights; the object owns the device copies
            g_layer = g_obj.layer
            dest = t2_res if t2_fam == 0 else t2_res.setdefault("family3_matrix_core_gemv", {})
            for nb in (1, 4, 8, 16):
                xs = (torch.randn((nb, max(D, F, nq * d)), device="cuda") * 0.5).to(torch.bfloat16).view(torch.int16)
                oq = torch.empty((nb, nqkv), dtype=torch.int16, device="cuda")
                oh = torch.empty((nb, D), dtype=torch.float32, device="cuda")
                og = torch.empty((nb, F), dtype=torch.int16, device="cuda")
                res = torch.zeros((nb, D), dtype=torch.float32, device="cuda")
                xd = xs[:, :D].contiguous()
                xa = xs[:, :nq * d].contiguous()
                xf = xs[:, :F].contiguous()

                def gemv_pass():
                    pkd.gemv_rows(g_layer.w_qkv, xd, 1, nb, oq, 1)
                    pkd.gemv_rows(g_layer.w_o, xa, 1, nb, oh, 0, residual=res)
                    pkd.gemv_rows(g_layer.w_gate_up, xd, 1, nb, og, 1, silu_pair=True)
                    pkd.gemv_rows(g_layer.w_down, xf, 1, nb, oh, 0, residual=res)
                for _ in range(3):
                    gemv_pass()
                med, p10, p90 = timed(gemv_pass, max(args.steps, 10), True)
                byt = wbytes + nb * 2 * (D + nq * d + D + F) + nb * (2 * nqkv + 8 * D + 2 * F + 8 * D)
                dest[f"B{nb}"] = {"us": round(med, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2),
                                  "bytes": int(byt), "GB_s": round(byt / med / 1e3, 1),
                                  "hbm_frac": round(byt / med / 1e3 / HBM_PEAK_GBS, 4)}
    # Output head over a tied embedding (151,936 x 2,048 bf16, 593.5 MiB): the
    # dense head at batch 1 against the candidate-row head, whose rows carry
    # trie-shaped lists of 1..28 candidates, cold.
    head_res = None
    if not args.no_head:
        V, HD, HC = wl.HEAD_VOCAB, wl.HEAD_HIDDEN, wl.HEAD_MAX_CAND
        gh = torch.Generator(device="cuda").manual_seed(7)
        Wh = torch.empty((V, HD), dtype=torch.int16, device="cuda")
        for i in range(0, V, 16384):
            blk = torch.randn((min(16384, V - i), HD), generator=gh, device="cuda") * 0.02
            Wh[i:i + blk.shape[0]] = blk.to(torch.bfloat16).view(torch.int16)
        Mh = pkd.make_matrix(Wh, V, HD, 1, 1.0, 0)
        head_res = {"vocab": V, "hidden": HD, "max_cand": HC, "dtype": "bf16", "matrix_bytes": V * HD * 2}
        for nb in (1, 64, 512):
            xh = (torch.randn((nb, HD), generator=gh, device="cuda")).to(torch.bfloat16).view(torch.int16)
            cand, n_cand = wl.head_candidates(nb, V, HC, 1000 + nb)
            cd, nd = torch.from_numpy(cand).cuda(), torch.from_numpy(n_cand).cuda()
            yh = torch.empty((nb, HC), device="cuda")
            gbytes = int(n_cand.sum()) * HD * 2 + nb * HD * 2 + int(n_cand.sum()) * 4 + nb * HC * 4 + nb * 4
            for _ in range(3):
                pkd.gemv_gather_rows(Mh, xh, 1, nb, cd, nd, HC, yh)
            med, p10, p90 = timed(lambda: pkd.gemv_gather_rows(Mh, xh, 1, nb, cd, nd, HC, yh),
                                  max(args.steps, 10), True)
            ent = {"gathered_us": round(med, 2), "gathered_p10_us": round(p10, 2), "gathered_p90_us": round(p90, 2),
                   "gathered_bytes": gbytes, "gathered_GB_s": round(gbytes / med / 1e3, 1),
                   "mean_candidates": round(float(n_cand.mean()), 2)}
            if nb == 1:
                yd = torch.empty((nb, V), device="cuda")
                for _ in range(3):
                    pkd.gemv_rows(Mh, xh, 1, nb, yd, 0)
                dmed, _, _ = timed(lambda: pkd.gemv_rows(Mh, xh, 1, nb, yd, 0), max(args.steps, 10), True)
                dbytes = V * HD * 2 + HD * 2 + V * 4
                ent.update({"dense_us": round(dmed, 2), "dense_bytes": dbytes,
                            "dense_GB_s": round(dbytes / dmed / 1e3, 1),
                            "dense_hbm_frac": round(dbytes / dmed / 1e3 / HBM_PEAK_GBS, 4),
                            "speedup_vs_dense": round(dmed / med, 1)})
                del yd
            head_res[f"B{nb}"] = ent
        del Wh, Mh
    # Prefill of one 2,662-token prompt in 256-token chunks through the same
    # layer shape: the chunk as one step (matrix-core projections, shared-tile
    # attention) against the same 256 tokens one step each (vector GEMV at
    # batch 1), and the chunk's attention with shared tiles against per-row.
    prefill_res = None
    if not args.no_prefill and w.w_dtype == 1 and F:
        lname = "7b" if D == 3584 else "0.6b"
        prefill_res = {"layer": lname, "prompt_tokens": 2662, "chunk_tokens": 256, "attn_chunk_pages": 8}
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
            with torch.cuda.stream(gstream):
                pkd.decode_step(layp.layer, poolp.handle, rows_p, xp, yp, wsp, stream=gstream)
                gp = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gp, stream=gstream):
                    pkd.decode_step(layp.layer, poolp.handle, rows_p, xp, yp, wsp, stream=gstream)
                for _ in range(args.warmup):
                    gp.replay()
                g0.record(gstream)
                for _ in range(args.steps):
                    gp.replay()
                g1.record(gstream)
            torch.cuda.synchronize()
            us_chunk = g0.elapsed_time(g1) / args.steps * 1e3
            pkd.pkd_pool_check(poolp.handle)
            # the same 256 tokens one step each, in order (vector family at batch 1)
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
            e0.record(stream)
            token_by_token()
            e1.record(stream)
            torch.cuda.synchronize()
            us_tokens = e0.elapsed_time(e1) * 1e3
            # attention of the chunk alone (appends already in the pool): shared tiles against per-row
            qa = (torch.randn((nP, nq, d), device="cuda")).to(torch.bfloat16).view(torch.int16)
            oa = torch.empty((nP, nq, d), dtype=torch.int16, device="cuda")
            wsa = H.aligned_empty(pkd.pkd_attn_workspace_bytes(poolp.handle, nq, nP))
            rows_row = pkd.make_rows(sp, pp, True)  # no append: the per-row kernels, tiles off
            att_t, _, _ = timed(lambda: pkd.paged_attn_decode(poolp.handle, rows_p, nq, qa, None, None, oa, 1, wsa),
                                max(args.steps, 10), False)
            att_r, _, _ = timed(lambda: pkd.paged_attn_decode(poolp.handle, rows_row, nq, qa, None, None, oa, 1, wsa),
                                max(args.steps, 10), False)
            prefill_res[f"pos{p0}"] = {
                "us_chunk_step": round(us_chunk, 1), "tokens_per_s": round(nP / us_chunk * 1e6),
                "us_token_by_token": round(us_tokens, 1), "speedup_vs_token_by_token": round(us_tokens / us_chunk, 1),
                "attention_us_shared_tiles": round(att_t, 2), "attention_us_per_row": round(att_r, 2)}
            del wp, poolp, layp, lay1
    del flush, flush_sum

    # ---------------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        nr = min(args.cpu_rows, B)
        rws = np.arange(nr)
        seqs = np.unique(w.seq[rws])
        hk, hv = wl.history_lists(w, seqs)
        hist = orc.History(hk, hv, w.kv_dtype, nkv, d)
        lay = wl.layer_dict(w)
        xs = w.x[:nr].cpu().numpy()
        print(f"[bench] cpu baseline: oracle on {nr} rows, {orc.threads()} threads", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        orc.decode_step(lay, hist, w.seq[rws], w.pos[rws], xs)
        t1 = time.perf_counter()
        per_step = (t1 - t0) / nr * B
        cpu = {"value": round(total_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": orc.threads(),
               "kind": "oracle", "us_per_step": round(per_step * 1e6, 1),
               "sample": f"fp64 oracle decode step of the first {nr} of {B} rows ({t1 - t0:.1f} s), "
                         f"time per row x {B} rows"}

    line = {
        "metric": "decode-step us and achieved HBM GB/s (% of peak), paged attn + GEMV",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "us_per_step": round(ms_step * 1e3, 2),
        "us_per_step_eager": round(ms_eager * 1e3, 2),
        "us_per_step_norm_rope": round(ms_step_nr * 1e3, 2),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {0: "f32", 1: "bf16", 2: "fp8"}[w.w_dtype], "data": "synthetic",
        "config": {"workload": w.name, "rows": B, "hidden": D, "q_heads": nq, "kv_heads": nkv, "head_dim": d,
                   "ffn": F, "page_tokens": 32, "kv_tokens_unique": int(kv_tokens),
                   "projection_family": int(fam), "parallelism": "none (1 GPU)"},
        "step_bytes": int(total_bytes),
        "kernels": kernels,
        "roofline": roofline,
        "t1_attention": t1_res,
        "t2_gemv": t2_res,
        "output_head": head_res,
        "prefill": prefill_res,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
