"""Pins for the pack oracle: a hand-worked tree, closed forms, parent closure."""
import numpy as np
import pytest

from oracle import pack_ref, parents_ref, visible_intervals_ref, visible_ref
from specgen import gen_structure, get_config, small_config


def _rand_structure(rng, n_trees, tmax, bmax, wmax):
    T = rng.integers(1, tmax + 1, size=n_trees)
    nb = rng.integers(0, bmax + 1, size=n_trees)
    anchors = np.concatenate([rng.integers(0, T[t], size=nb[t]) for t in range(n_trees)]).astype(int)
    widths = rng.integers(1, wmax + 1, size=int(nb.sum()))
    return T, nb, anchors, widths


def test_hand_worked_tree(golden):
    g = golden("pack_tiny.json")
    lay = pack_ref(**g["inputs"])
    for key, val in g["expected"].items():
        got = lay[key]
        if isinstance(got, np.ndarray):
            assert got.tolist() == val, key
        else:
            assert got == val, key
    mask = visible_ref(lay)
    for r, vis in g["visible"].items():
        assert np.flatnonzero(mask[int(r)]).tolist() == vis


def test_fig4_readout_rule(golden):
    g = golden("fig4_readout.json")
    T = len(g["trunk_tokens"])
    lay = pack_ref([T], [1], [g["anchor"]], [len(g["branch_tokens"])])
    token_of_row = list(g["trunk_tokens"]) + list(g["branch_tokens"][:-1])  # terminal sample has no row
    assert lay["n_rows"] == len(token_of_row)
    for s, tok in enumerate(g["branch_tokens"]):
        assert token_of_row[lay["step_pred_row"][s]] == g["expected_query_token_for_step"][tok]
        # a token's own row is never its readout row
        if lay["step_sample_row"][s] >= 0:
            assert lay["step_pred_row"][s] != lay["step_sample_row"][s]


@pytest.mark.parametrize("seed", range(6))
def test_closed_forms_and_parent_closure(seed):
    rng = np.random.default_rng(100 + seed)
    T, nb, anchors, widths = _rand_structure(rng, n_trees=1 + seed % 3, tmax=40, bmax=7, wmax=6)
    lay = pack_ref(T, nb, anchors, widths)
    N = int(T.sum() + (widths - 1).sum())
    R = int(widths.sum())
    assert lay["n_rows"] == N and lay["n_steps"] == R
    mask = visible_ref(lay)
    # the two-interval rule equals the parent closure, row by row
    for r in range(N):
        assert np.array_equal(np.flatnonzero(mask[r]), np.sort(visible_intervals_ref(lay, r)))
    # popcount equals the causal-pair count: trunk triangles plus branch rows
    P = sum(int(t) * (int(t) + 1) // 2 for t in T)
    P += sum(int(anchors[b]) + 1 + i for b in range(len(anchors)) for i in range(1, int(widths[b])))
    assert int(mask.sum()) == P
    # semantic position equals depth in the tree
    par = parents_ref(lay)
    depth = np.zeros(N, int)
    for r in range(N):
        depth[r] = 0 if par[r] < 0 else depth[par[r]] + 1
    assert np.array_equal(depth, lay["row_pos"])
    # every step's readout row is its sample's parent; the sample row is never read
    for s in range(R):
        if lay["step_sample_row"][s] >= 0:
            assert par[lay["step_sample_row"][s]] == lay["step_pred_row"][s]
    # rows are a permutation grouped by tree; branch rows of b are contiguous
    for b in range(len(anchors)):
        rows = np.flatnonzero(lay["row_branch"] == b)
        assert rows.tolist() == list(range(lay["branch_off"][b], lay["branch_off"][b] + widths[b] - 1))


def test_duplicate_anchors_and_one_token_branches():
    lay = pack_ref([10], [4], [3, 3, 3, 9], [1, 4, 2, 1])
    assert lay["n_rows"] == 10 + 0 + 3 + 1 + 0
    assert lay["n_steps"] == 8
    # both one-token branches have one step, read from their anchor rows, no packed row
    assert lay["step_pred_row"][0] == 3 and lay["step_sample_row"][0] == -1
    assert lay["step_pred_row"][7] == 9 and lay["step_sample_row"][7] == -1
    # the duplicate-anchor branches never see each other
    mask = visible_ref(lay)
    r1 = np.flatnonzero(lay["row_branch"] == 1)
    r2 = np.flatnonzero(lay["row_branch"] == 2)
    assert not mask[np.ix_(r1, r2)].any() and not mask[np.ix_(r2, r1)].any()


def test_no_branches_is_plain_causal():
    lay = pack_ref([7], [0], [], [])
    assert lay["n_rows"] == 7 and lay["n_steps"] == 0
    assert np.array_equal(visible_ref(lay), np.tril(np.ones((7, 7), bool)))


@pytest.mark.parametrize("bad", [
    dict(trunk_len=[5], n_branches=[1], anchors=[5], branch_len=[2]),     # anchor == T
    dict(trunk_len=[5], n_branches=[1], anchors=[-1], branch_len=[2]),    # negative anchor
    dict(trunk_len=[5], n_branches=[1], anchors=[1], branch_len=[0]),     # width 0
    dict(trunk_len=[0], n_branches=[0], anchors=[], branch_len=[]),       # empty trunk
    dict(trunk_len=[5], n_branches=[2], anchors=[1], branch_len=[2]),     # count mismatch
])
def test_invalid_inputs_rejected(bad):
    with pytest.raises(ValueError):
        pack_ref(**bad)


@pytest.mark.parametrize("name", ["tiny", "gqa8b", "batched", "stress"])
def test_workload_structures(name):
    cfg = get_config(name)
    s = gen_structure(cfg)
    lay = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    assert lay["n_rows"] == int(s["trunk_len"].sum() + (s["branch_len"] - 1).sum())
    assert lay["n_steps"] == int(s["branch_len"].sum())
    if name == "gqa8b":
        assert (lay["n_rows"], lay["n_steps"]) == (7936, 4096)
        assert len(set(s["anchors"].tolist())) == 256      # drawn without replacement
    if name == "batched":
        assert (lay["n_rows"], lay["n_steps"]) == (23552, 8192)
        assert lay["tree_off"].tolist() == [2944 * t for t in range(9)]
    if name == "tiny":
        assert (lay["n_rows"], lay["n_steps"]) == (76, 16)
    assert s["anchors"].min() >= cfg.anchor_lo and s["anchors"].max() < cfg.trunk


def test_generator_is_deterministic():
    cfg = small_config("gqa8b", trunk=100, branches=7)
    a, b = gen_structure(cfg), gen_structure(cfg)
    for k in a:
        assert np.array_equal(a[k], b[k])
