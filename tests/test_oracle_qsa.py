"""Pins of the sparse-attention oracle (branch-consistent indexer groups) against things
other than itself: the Figure 4 example, each branch scored as its own sequence, the
full-attention oracle, closed forms and isolation."""
import numpy as np
import pytest

from oracle import pack_ref, tree_attn_ref
from oracle.qsa_ref import (qsa_attn_ref, qsa_brute_force_branch_ref, qsa_causal_ref, qsa_group_keys,
                            qsa_history_ref, qsa_pick, qsa_row_structure)


def _layout(trunks, anchors_per_tree, widths):
    T = np.array(trunks, np.int32)
    nb = np.array([len(a) for a in anchors_per_tree], np.int32)
    a = np.array([x for t in anchors_per_tree for x in t], np.int32)
    return pack_ref(T, nb, a, np.array(widths, np.int32))


def _inputs(N, hq, hkv, D, DI, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, hq, D))
    k = rng.standard_normal((N, hkv, D))
    v = rng.standard_normal((N, hkv, D))
    qi = rng.standard_normal((N, hkv, DI))
    ki = rng.standard_normal((N, hkv, DI))
    return q, k, v, qi, ki


def test_fig4_example_structure(golden):
    """Groups, tails and branch-specific keys of the caption's example."""
    gd = golden("fig4_sparse_groups.json")
    G = gd["group_size"]
    trunk, branch, a = gd["trunk"], gd["branch"], gd["anchor"]
    lay = _layout([len(trunk)], [[a]], [len(branch)])
    tok = {}
    for j, name in enumerate(trunk):
        tok[j] = name
    for i in range(len(branch) - 1):
        tok[int(lay["branch_off"][0]) + i] = branch[i]
    for s, want in enumerate(gd["steps"]):
        r = int(lay["step_pred_row"][s])
        assert tok[r] == want["query_token"]
        hist = qsa_history_ref(lay, r)
        t = len(hist) - 1
        n_c, tail = qsa_row_structure(t, G)
        groups = [[tok[int(hist[p])] for p in range(G * j, G * j + G)] for j in range(n_c)]
        assert groups == want["complete_groups"]
        assert [tok[int(hist[p])] for p in tail] == want["tail"]
        # a group is branch-specific iff it holds a position past the anchor
        assert [bool(G * j + G - 1 > a) for j in range(n_c)] == want["branch_specific"]
    for want in gd["trunk_rows"]:
        r = trunk.index(want["query_token"])
        hist = qsa_history_ref(lay, r)
        n_c, tail = qsa_row_structure(len(hist) - 1, G)
        assert [[tok[int(hist[p])] for p in range(G * j, G * j + G)] for j in range(n_c)] == want["complete_groups"]
        assert [tok[int(hist[p])] for p in tail] == want["tail"]


def test_fig4_branch_specific_key_differs_from_trunk_key(golden):
    """The group completed by 'with' averages the branch token's indexer key, not the
    trunk token that follows the anchor."""
    gd = golden("fig4_sparse_groups.json")
    G = gd["group_size"]
    lay = _layout([len(gd["trunk"])], [[gd["anchor"]]], [len(gd["branch"])])
    N = lay["n_rows"]
    ki = np.zeros((N, 1, 4))
    for r in range(N):
        ki[r, 0, r % 4] = r + 1.0                       # distinct per row
    row_with = int(lay["branch_off"][0])
    hb = qsa_history_ref(lay, row_with)
    ht = qsa_history_ref(lay, 7)                        # trunk row 'next'
    kb = qsa_group_keys(ki[hb], G)[1, 0]
    kt = qsa_group_keys(ki[ht], G)[1, 0]
    # by hand: mean of rows 4, 5, 6 and the branch row (trunk: rows 4, 5, 6, 7)
    assert np.allclose(kb, (ki[4, 0] + ki[5, 0] + ki[6, 0] + ki[row_with, 0]) / 4, rtol=0, atol=0)
    assert np.allclose(kt, (ki[4, 0] + ki[5, 0] + ki[6, 0] + ki[7, 0]) / 4, rtol=0, atol=0)
    assert not np.allclose(kb, kt)


@pytest.mark.parametrize("G,top_k", [(4, 2), (4, 1), (8, 3), (1, 5), (3, 2)])
def test_packed_equals_each_branch_as_its_own_sequence(G, top_k):
    """[SpecOPD notes page, "Checks, negative controls, and limits"]: packed scoring equals
    independent causal scoring. Anchors at group edges (a = 0, G-1, G, 2G-1), duplicates,
    a one-token branch, two trees."""
    lay = _layout([37, 21], [[0, G - 1, G, 2 * G - 1, 2 * G - 1, 30, 36], [5, 20, 13]],
                  [6, 5, 1, 9, 4, 7, 3, 8, 2, 6])
    N = lay["n_rows"]
    q, k, v, qi, ki = _inputs(N, 4, 2, 16, 8, seed=G * 10 + top_k)
    out, picks = qsa_attn_ref(lay, q, k, v, qi, ki, G, top_k, 10000.0)
    worst = 0.0
    for b in range(lay["n_branches"]):
        rows, ob, pb = qsa_brute_force_branch_ref(lay, q, k, v, qi, ki, b, G, top_k, 10000.0)
        worst = max(worst, float(np.abs(out[rows] - ob).max()))
        assert np.array_equal(picks[rows], pb)
    for t in range(2):
        lo = int(lay["tree_off"][t])
        hi = lo + [37, 21][t]
        ot, pt = qsa_causal_ref(q[lo:hi], k[lo:hi], v[lo:hi], qi[lo:hi], ki[lo:hi], G, top_k, 10000.0)
        worst = max(worst, float(np.abs(out[lo:hi] - ot).max()))
        assert np.array_equal(picks[lo:hi], pt)
    assert worst < 1e-12


def test_top_k_covering_every_group_is_full_attention():
    """With top_k at least the number of groups, every history key is read: the result is
    the full tree attention of the packed tree."""
    lay = _layout([40], [[3, 17, 17, 39]], [5, 7, 2, 4])
    q, k, v, qi, ki = _inputs(lay["n_rows"], 4, 2, 16, 8, seed=3)
    out, _ = qsa_attn_ref(lay, q, k, v, qi, ki, 4, 64, 10000.0)
    full = tree_attn_ref(lay, q, k, v, 10000.0)
    assert np.abs(out - full).max() < 1e-12


def test_closed_form_uniform_scores_and_known_ranking():
    """K = 0 makes attention a plain mean over the read keys. Indexer keys constant within a
    group (c_j times a fixed vector) and queries equal to that vector rank the groups by c_j,
    so the read set is known in closed form: the top_k groups by c_j plus the causal tail."""
    G, top_k, D, DI = 4, 3, 8, 6
    lay = _layout([45], [[9, 22, 44]], [6, 9, 3])
    N = lay["n_rows"]
    rng = np.random.default_rng(11)
    u = rng.standard_normal(DI)
    c = rng.permutation(20).astype(np.float64) + 1.0      # distinct group weights
    ki = np.zeros((N, 1, DI))
    qi = np.tile(u, (N, 1, 1))
    v = rng.standard_normal((N, 1, D))
    q = rng.standard_normal((N, 2, D))
    k = np.zeros((N, 1, D))
    for r in range(N):                                    # a token's position is the same in
        ki[r, 0] = c[int(lay["row_pos"][r]) // G] * u     # every history that holds it
    out, picks = qsa_attn_ref(lay, q, k, v, qi, ki, G, top_k, 10000.0)
    for r in range(N):
        hist = qsa_history_ref(lay, r)
        t = len(hist) - 1
        n_c = (t + 1) // G
        want = np.sort(np.argsort(-c[:n_c], kind="stable")[:top_k]) if n_c > top_k else np.arange(n_c)
        got = picks[r, 0][picks[r, 0] >= 0]
        assert np.array_equal(got, want), r
        pos = np.concatenate([(G * want[:, None] + np.arange(G)).ravel(), np.arange(n_c * G, t + 1)])
        mean = v[hist[pos], 0].mean(axis=0)
        assert np.abs(out[r] - mean[None, :]).max() < 1e-12


def test_pick_rule_ties_and_counts():
    s = np.array([3.0, 1.0, 3.0, 2.0, 3.0])
    assert qsa_pick(s, 2).tolist() == [0, 2]               # ties: lower index first
    assert qsa_pick(s, 4).tolist() == [0, 2, 3, 4]
    assert qsa_pick(s, 9).tolist() == [0, 1, 2, 3, 4]       # fewer groups than k: all
    rng = np.random.default_rng(2)
    for _ in range(50):
        x = rng.standard_normal(rng.integers(1, 40))
        kk = int(rng.integers(1, 10))
        sel = qsa_pick(x, kk)
        rest = np.setdiff1d(np.arange(len(x)), sel)
        assert len(sel) == min(kk, len(x))
        if len(rest):
            assert x[sel].min() >= x[rest].max()           # every pick outranks every other group


def test_isolation_from_other_branches():
    """Changing every token outside a branch row's history changes neither its output nor
    its picks ([SpecOPD notes page, "Checks, negative controls, and limits"])."""
    G, top_k = 4, 2
    lay = _layout([30], [[7, 7, 15, 29]], [6, 6, 5, 4])
    N = lay["n_rows"]
    q, k, v, qi, ki = _inputs(N, 4, 2, 16, 8, seed=5)
    out, picks = qsa_attn_ref(lay, q, k, v, qi, ki, G, top_k, 10000.0)
    rng = np.random.default_rng(6)
    for b in range(lay["n_branches"]):
        mine = np.flatnonzero(lay["row_branch"] == b)
        keep = set(qsa_history_ref(lay, mine[-1]).tolist())
        other = np.array([r for r in range(N) if r not in keep])
        x = [a.copy() for a in (q, k, v, qi, ki)]
        for a in x:
            a[other] = rng.standard_normal(a[other].shape)
        o2, p2 = qsa_attn_ref(lay, *x, G, top_k, 10000.0, rows=mine)
        assert np.array_equal(o2, out[mine]) and np.array_equal(p2, picks[mine])
