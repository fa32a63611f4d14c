"""Host-side pieces of bench.py that its reported figures rest on: the causal-pair count
behind the attention roofline (against the oracle's parent-chain visibility), the keying
of measured traffic by source hash and workload, and the counter summary of a
rocprofv3 database. No GPU."""
import importlib.util
import json
import os
import sqlite3

import numpy as np
import pytest

from oracle import pack_ref, visible_ref
from specgen import CONFIGS, gen_structure

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("seed", range(6))
def test_causal_pairs_match_oracle_visibility(bench, seed):
    """Pairs counted from the closed form equal the visible (row, key) pairs of the
    oracle's mask, which walks every row's parent chain (trees, duplicate anchors,
    one-step branches, anchors at 0 and T-1)."""
    rng = np.random.default_rng(seed)
    n_trees = int(rng.integers(1, 4))
    T = rng.integers(1, 60, size=n_trees).astype(np.int32)
    nb = rng.integers(0, 7, size=n_trees).astype(np.int32)
    anchors = np.concatenate([rng.integers(0, t, size=b) for t, b in zip(T, nb)]).astype(np.int32)
    widths = rng.integers(1, 12, size=int(nb.sum())).astype(np.int32)
    if len(anchors):
        anchors[0] = 0
        anchors[-1] = T[-1] - 1 if nb[-1] else anchors[-1]
    s = dict(trunk_len=T, n_branches=nb, anchors=anchors, branch_len=widths)
    lay = pack_ref(T, nb, anchors, widths)
    assert bench.causal_pairs(s) == int(visible_ref(lay).sum())


def test_causal_pairs_workload_trunk_part(bench):
    """gqa8b: the trunk triangle is T(T+1)/2 and every branch row of branch b sees
    a_b + 1 trunk rows plus its own branch prefix."""
    s = gen_structure(CONFIGS["gqa8b"])
    T = int(s["trunk_len"][0])
    a = s["anchors"].astype(np.int64)
    w = s["branch_len"].astype(np.int64)
    brute = sum(int(w[b] - 1) * int(a[b] + 1) + sum(range(1, int(w[b]))) for b in range(len(a)))
    assert bench.causal_pairs(s) == T * (T + 1) // 2 + brute


def test_measured_traffic_keyed_by_source_and_workload(bench, tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"tree_attn": {"source_hash": "abc", "workload": "stress",
                                              "bytes_per_launch": 123.0}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("tree_attn", "abc", "stress") == 123.0
    assert bench.measured_traffic("tree_attn", "abd", "stress") is None      # kernel source changed
    assert bench.measured_traffic("tree_attn", "abc", "gqa8b") is None       # another workload
    assert bench.measured_traffic("e2etv_fused", "abc", "stress") is None    # never measured
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("tree_attn", "abc", "stress") is None


def test_source_hash_covers_shared_header(bench):
    """The committed traffic of every mark is keyed by its sources and common.h."""
    h1 = bench.source_hash("attn.hip", "rope.hip")
    assert h1 == bench.source_hash("attn.hip", "rope.hip") and len(h1) == 16
    assert h1 != bench.source_hash("rope.hip")
    for mark, (subs, srcs) in bench.MARK_KERNELS.items():
        for src in srcs:
            assert os.path.exists(os.path.join(ROOT, "tree_attention_spec_amd", "csrc", src)), (mark, src)


def test_summarize_pmc_means_per_kernel(bench, tmp_path):
    """Per-kernel means over dispatches, read through the same join the profiler's
    database offers (kernels x pmc_events)."""
    db = tmp_path / "pmc_results.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (dispatch_id integer, name text)")
    con.execute("create table pmc_events (dispatch_id integer, counter_name text, counter_value real)")
    con.executemany("insert into kernels values (?, ?)", [(1, "k_a"), (2, "k_a"), (3, "k_b")])
    con.executemany("insert into pmc_events values (?, ?, ?)",
                    [(1, "FETCH_SIZE", 10.0), (2, "FETCH_SIZE", 30.0), (3, "FETCH_SIZE", 5.0),
                     (3, "WRITE_SIZE", 7.0)])
    con.commit()
    con.close()
    out = bench.summarize_pmc([str(db)])
    assert out["k_a"]["FETCH_SIZE"] == {"dispatches": 2, "mean": 20.0}
    assert out["k_b"]["FETCH_SIZE"]["mean"] == 5.0 and out["k_b"]["WRITE_SIZE"]["mean"] == 7.0
