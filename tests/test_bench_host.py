"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop
accounting behind `value` and `roofline`, the gating of committed HBM-traffic
figures by kernel source, and the one-GPU refusal."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

ELEM = {0: 4, 1: 2, 2: 1}  # f32, bf16, fp8 bytes


def _tiny():
    """Three rows, two sequences, one physical page shared as a prefix.

    Sequence 0 (pages 7, 3) has two rows, at positions 40 and 41 (contexts of
    41 and 42 tokens); sequence 1 (page 7 only, shared) has one row at
    position 5 (6 tokens).  Unique (page, slot) pairs read: page 7 slots
    0..31 and page 3 slots 0..9, so 42 tokens; page reads per row: 2, 2, 1.
    """
    tables = np.array([[7, 3], [7, -1]], dtype=np.int32)
    return SimpleNamespace(n_rows=3, hidden=64, n_q=4, n_kv=2, head_dim=16, ffn=128,
                           w_dtype=1, kv_dtype=1, act_dtype=1, tables=tables,
                           seq=np.array([0, 0, 1], dtype=np.int32), pos=np.array([40, 41, 5], dtype=np.int32))


def test_unique_kv_tokens_count_shared_pages_once():
    _, _, kv_tokens = bench.step_bytes(_tiny(), ELEM)
    assert kv_tokens == 42


def test_attention_bytes_and_flops_by_hand():
    st, flops, _ = bench.step_bytes(_tiny(), ELEM)
    # K and V of 42 tokens x 2 kv heads x 16 dims in bf16: 42 * 2 * 2 * 16 * 2 = 5,376
    # q in and out of 3 rows x 4 heads x 16 dims in bf16: 3 * 4 * 16 * 4 = 768
    # table entries 4 * (2 + 2 + 1) = 20, row seq/pos 8 * 3 = 24
    assert st["attention"] == 5376 + 768 + 20 + 24
    # q.k and p.v: 4 flops per (q head, dim, token) over 41 + 42 + 6 tokens
    assert flops["attention"] == 4 * 4 * 16 * 89


def test_projection_flops_and_gate_up_bytes_by_hand():
    st, flops, _ = bench.step_bytes(_tiny(), ELEM)
    assert flops["qkv"] == 2 * 3 * 128 * 64       # (4 + 2 * 2) heads x 16 = 128 outputs
    assert flops["wo"] == 2 * 3 * 64 * 64
    assert flops["gate_up"] == 2 * 3 * 256 * 64   # gate and up: 2 x 128 outputs
    assert flops["down"] == 2 * 3 * 64 * 128
    # gate/up: weights 256 x 64 bf16, x of 3 rows x 64 bf16, silu output 3 x 128 bf16
    assert st["gate_up"] == 32768 + 384 + 768


def test_implementation_passes_not_counted():
    """The bf16 cast of x, the bf16 copy of h and K-split partial sums are the
    implementation's, not the method's: only weights, inputs, outputs and
    residual reads are counted."""
    st, _, _ = bench.step_bytes(_tiny(), ELEM)
    assert "cast" not in st
    # W_o: weights 64 x 64 bf16, attn 3 x 64 bf16, residual x read and h written in f32
    assert st["wo"] == 64 * 64 * 2 + 3 * 64 * 2 + 3 * 64 * 4 * 2
    # qkv: weights 128 x 64, x in the activation dtype, qkv out
    assert st["qkv"] == 128 * 64 * 2 + 3 * 64 * 2 + 3 * 128 * 2
    # the append writes each row's key and value once
    assert st["append"] == 3 * 2 * 2 * 16 * 2


def test_stage_roofline():
    # attention: HBM; fp8 matrix cores for family 2, bf16 for families 1 and 3, vector ALU for 0
    assert bench.stage_peak("attention", -1, 1) == ("hbm", None)
    assert bench.stage_peak("gate_up", 2, 2) == ("mfma", 5000.0)
    assert bench.stage_peak("gate_up", 1, 2) == ("mfma", 2500.0)
    assert bench.stage_peak("qkv", 3, 1) == ("mfma", 2500.0)
    assert bench.stage_peak("qkv", 0, 1) == ("alu", 157.3)
    # 8 GB at 8 TB/s = 1 ms; 5 PFLOP at 2.5 PF = 2 s: the larger wins
    assert abs(bench.ideal_us(8e9, 0, None) - 1e3) < 1e-9
    assert abs(bench.ideal_us(8e9, 5e15, 2500.0) - 2e6) < 1e-6
    assert abs(bench.ideal_us(8e9, 1e9, 2500.0) - 1e3) < 1e-9


def test_traffic_figure_used_only_for_its_sources(monkeypatch):
    got = bench.measured_traffic("gate_up", "7b-b768-prefix-bf16", 1)
    path = os.path.join(ROOT, "profiles", "gate_up_7b-b768-prefix-bf16.traffic.txt")
    kv = {}
    with open(path) as fh:
        for line in fh:
            if not line.startswith("#") and ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv["source_sha256"] == bench.source_hash("gate_up", 1):
        assert got == int(kv["traffic_bytes_per_launch"])
    else:  # the kernel changed since the counters were taken: no figure
        assert got is None
    monkeypatch.setattr(bench, "source_hash", lambda stage, family: "0" * 64)
    assert bench.measured_traffic("gate_up", "7b-b768-prefix-bf16", 1) is None
    assert bench.measured_traffic("gate_up", "no-such-workload", 1) is None


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
