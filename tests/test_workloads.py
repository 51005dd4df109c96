"""The seeded input recipes (tests/workloads.py) produce the structure they
state: shared and private pages, length mixes, positions and history.  Both
the oracle and the GPU path consume these inputs, so a recipe that drifted
would weaken every parity and bench figure built on it.  Reduced row counts
keep the CPU suite fast; the structure does not depend on them."""
import numpy as np
import torch

import workloads as wl


def _listed_pages(w):
    out = []
    for s in range(w.max_seqs):
        out.extend(int(p) for p in w.tables[s][: int(w.counts[s])])
    return out


def test_b768_prefix_structure():
    n = 96
    w = wl.make("7b-b768-prefix-bf16", "cpu", n=n, with_weights=False)
    lens = w.pos.astype(np.int64) + 1
    assert np.array_equal(w.seq, np.arange(n))
    assert lens.min() >= 129 and lens.max() <= 256          # 128-token prompt + U{1..128}
    assert np.array_equal(w.hist_len, w.pos)                 # history = tokens before the row's own
    assert w.max_pages_per_seq == 8 and np.all(w.counts[:n] == 8)
    assert w.num_pages == 2 + 6 * n
    shared = w.tables[:n, :2]
    assert np.all(shared == shared[0])                       # two physically shared prompt pages
    private = w.tables[:n, 2:8].ravel()
    assert len(set(private.tolist())) == 6 * n               # every private page listed once
    assert not set(private.tolist()) & set(shared[0].tolist())
    assert 0 <= min(_listed_pages(w)) and max(_listed_pages(w)) < w.num_pages
    # the 90-token common prefix holds the same keys and values in every sequence
    for s in (1, n // 2, n - 1):
        o = int(w.hist_off[s])
        assert torch.equal(w.hist_k[o:o + 90], w.hist_k[0:90])
        assert torch.equal(w.hist_v[o:o + 90], w.hist_v[0:90])
    assert not torch.equal(w.hist_k[int(w.hist_off[1]) + 100], w.hist_k[100])


def test_mixed_step_structure():
    nd, cr, long_max = 40, 12, 1400
    w = wl.make("0.6b-mixed-bf16", "cpu", n_decode=nd, chunk_rows=cr, long_max=long_max)
    lens = w.pos[:nd].astype(np.int64) + 1
    n_long = int(np.sum(lens >= 1000))
    assert n_long == round(0.2 * nd)
    assert np.all((lens >= 1000) & (lens <= long_max) | (lens >= 100) & (lens <= 200))
    assert np.array_equal(w.seq[:nd], np.arange(nd))
    # the prompt chunk: rows of one sequence at consecutive positions from 1024, history 1024
    assert np.all(w.seq[nd:] == nd) and np.array_equal(w.pos[nd:], 1024 + np.arange(cr))
    assert int(w.hist_len[nd]) == 1024 and int(w.counts[nd]) == (2662 + 31) // 32
    # the pool is exactly the pages needed, each listed once
    assert sorted(_listed_pages(w)) == list(range(w.num_pages))
    assert w.x.shape == (nd + cr, 1024)


def test_fp8_pool_structure():
    n, L = 16, 96
    w = wl.make("7b-b4096-fp8", "cpu", n=n, L=L, with_weights=False)
    assert w.kv_dtype == wl.FP8 and w.w_dtype == wl.FP8
    assert np.all(w.pos == L - 1) and np.array_equal(w.seq, np.arange(n))
    assert np.all(w.counts[:n] == (L + 31) // 32)
    assert sorted(_listed_pages(w)) == list(range(w.num_pages))
    assert w.k_scale > 0 and w.v_scale > 0


def test_recipes_are_seeded():
    a = wl.make("7b-b768-prefix-bf16", "cpu", n=8, with_weights=False)
    b = wl.make("7b-b768-prefix-bf16", "cpu", n=8, with_weights=False)
    c = wl.make("7b-b768-prefix-bf16", "cpu", seed=1, n=8, with_weights=False)
    assert np.array_equal(a.tables, b.tables) and torch.equal(a.x, b.x) and torch.equal(a.hist_k, b.hist_k)
    assert not np.array_equal(a.pos, c.pos) or not torch.equal(a.x, c.x)
