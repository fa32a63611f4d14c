"""GPU parity: spec_tree_pack must equal the oracle's pack bit for bit."""
import numpy as np
import pytest

from _util import Case, say
from oracle import pack_ref
from specgen import CONFIGS, gen_structure

pytestmark = pytest.mark.gpu

COMPARED = ["tree_off", "row_tree", "row_branch", "row_anchor", "row_pos", "row_depth",
            "row_trunk_hi", "row_branch_lo", "branch_tree", "branch_anchor", "branch_len",
            "branch_off", "step_off", "branch_order", "step_branch", "step_pred_row",
            "step_sample_row"]


def _pack_gpu(s):
    import torch
    import tree_attention_spec_amd as tas
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    torch.cuda.synchronize()
    return tree, {k: v.cpu().numpy() for k, v in tree.arrays().items()}


def _check_groups(lay, it, groups):
    """The grouped schedule holds every block once, four to a group: consecutive blocks
    (in row order) of one tree's trunk rows or of one tree's branch rows, empty blocks
    padding a group's end, groups longest first (by their longest block), then empty
    groups."""
    n_trees = len(lay["tree_off"]) - 1
    assert groups.shape == (((len(it) + 3) // 4 + 2 * n_trees) * 4, 8)
    g = groups.reshape(-1, 4, 8)
    seen = []
    prev_cost = None
    done = False
    for grp in g:
        real = [b for b in grp if b[1] > b[0]]
        assert all(not b.any() for b in grp[len(real):])          # padding at the end, all zero
        if not real:
            done = True
            continue
        assert not done                                           # empty groups only at the end
        for a, b in zip(real, real[1:]):
            assert b[0] == a[1]                                   # consecutive rows
            assert b[2] == a[2]                                   # one tree
            assert (b[5] < b[6]) == (a[5] < a[6])                 # one kind: trunk or branch rows
        cost = max(int(b[7]) for b in real)
        assert prev_cost is None or cost <= prev_cost
        prev_cost = cost
        seen.extend(tuple(b) for b in real)
    assert sorted(seen) == sorted(tuple(b) for b in it)


def _check_items(lay, items):
    """The attention schedule covers every row once and every visible key of its rows."""
    n_items = lay["_n_attn_items"]
    it = items[:n_items * 8].reshape(-1, 8)
    _check_groups(lay, it, items[n_items * 8:].reshape(-1, 8))
    N = lay["n_rows"]
    seen = np.zeros(N, np.int64)
    for q0, q1, tk0, tk1, tfull, bk0, bk1, cost in it:
        assert 0 <= q0 < q1 <= N and q1 - q0 <= 32
        seen[q0:q1] += 1
        for r in range(q0, q1):
            t = lay["row_tree"][r]
            assert tk0 == lay["tree_off"][t]
            assert lay["row_trunk_hi"][r] < tk1                  # whole trunk prefix in range
            assert tfull <= lay["row_trunk_hi"][r] + 1           # unmasked tiles are visible
            if lay["row_branch"][r] >= 0:
                assert bk0 <= lay["row_branch_lo"][r] and r < bk1
            else:
                assert tk1 > r
        assert cost == (tk1 - tk0) + (bk1 - bk0)
    assert np.all(seen == 1)
    assert np.all(np.diff(it[:, 7]) <= 0)                        # longest first


def _compare(s, tag):
    say("pack parity: %s" % tag)
    ref = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    tree, got = _pack_gpu(s)
    assert tree.n_rows == ref["n_rows"] and tree.n_steps == ref["n_steps"]
    assert tree.max_branch_len == ref["max_branch_len"] and tree.max_pos == ref["max_pos"]
    for k in COMPARED:
        assert np.array_equal(got[k], ref[k]), k
    _check_items(dict(ref, _n_attn_items=tree.n_attn_items), got["attn_items"])


def test_pack_hand_worked(golden):
    g = golden("pack_tiny.json")
    s = {k: np.asarray(v, np.int32) for k, v in g["inputs"].items()}
    _compare(s, "hand-worked tree")


@pytest.mark.parametrize("seed", range(8))
def test_pack_random_trees(seed):
    rng = np.random.default_rng(seed)
    nt = int(rng.integers(1, 5))
    T = rng.integers(1, 200, size=nt)
    nb = rng.integers(0, 40, size=nt)
    anchors = np.concatenate([rng.integers(0, T[t], size=nb[t]) for t in range(nt)])
    widths = rng.integers(1, 65, size=int(nb.sum()))
    _compare(dict(trunk_len=T, n_branches=nb, anchors=anchors, branch_len=widths), "random %d" % seed)


def test_pack_edge_trees():
    cases = {
        "trunk only": ([37], [0], [], []),
        "single row": ([1], [1], [0], [1]),
        "all one-token": ([10], [4], [9, 0, 3, 3], [1, 1, 1, 1]),
        "anchor at ends": ([40], [3], [0, 39, 39], [64, 2, 33]),
        "empty trees between": ([5, 7, 5], [2, 0, 2], [1, 4, 0, 4], [3, 3, 16, 1]),
    }
    for tag, (T, nb, a, w) in cases.items():
        _compare(dict(trunk_len=np.array(T), n_branches=np.array(nb), anchors=np.array(a, np.int32),
                      branch_len=np.array(w, np.int32)), tag)


@pytest.mark.parametrize("name", ["tiny", "gqa8b", "long", "batched", "stress"])
def test_pack_workloads(name):
    _compare(gen_structure(CONFIGS[name]), name)


def test_pack_reuses_buffer_and_rejects_bad_input():
    import tree_attention_spec_amd as tas
    s = gen_structure(CONFIGS["tiny"])
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    tree2 = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"], mem=tree.mem)
    assert tree2.mem.data_ptr() == tree.mem.data_ptr()
    with pytest.raises(tas.SpecError):
        tas.spec_tree_pack([10], [1], [10], [2])
    with pytest.raises(tas.SpecError):
        tas.spec_tree_pack([10], [1], [3], [65])
