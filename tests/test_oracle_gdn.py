"""Pins of the GDN replay oracle: closed forms of one delta-rule token, the
ancestry of the short convolution on a hand-worked tree, and indexed replay
from checkpoints against each branch scored as its own sequence from the zero
state (which uses neither checkpoints nor the parent array)."""
import numpy as np
import pytest

from oracle import (
    ancestors_ref,
    conv_ancestry_ref,
    gdn_branch_brute_ref,
    gdn_checkpoints_ref,
    gdn_features_ref,
    gdn_replay_ref,
    gdn_step_ref,
    gdn_trunk_ref,
    pack_ref,
    silu,
    trunk_len_ref,
)


def _inputs(N, H, D, K, seed):
    g = np.random.default_rng(seed)
    x = [g.standard_normal((N, H, D)) for _ in range(3)]
    w = [0.5 * g.standard_normal((H, D, K)) for _ in range(3)]
    alpha = g.uniform(0.8, 1.0, size=(N, H))
    beta = g.uniform(0.1, 0.9, size=(N, H))
    return x, w, alpha, beta


def test_silu_values():
    assert silu(0.0) == 0.0
    assert np.isclose(silu(1.0), 1.0 / (1.0 + np.exp(-1.0)), rtol=0, atol=1e-15)
    x = np.linspace(-30, 30, 121)
    assert np.allclose(silu(x) - silu(-x), x, rtol=0, atol=1e-12)   # x s(x) + x s(-x) = x
    assert np.allclose(silu(np.array([40.0])), 40.0, rtol=1e-15)


def test_ancestors_hand_tree():
    # trunk 0..4; branch 0 at anchor 1 with y1, y2 (rows 5, 6); branch 1 at anchor 4 with y1 (row 7)
    lay = pack_ref([5], [2], [1, 4], [3, 2])
    anc = ancestors_ref(lay, 4)
    assert anc[0].tolist() == [0, -1, -1, -1]
    assert anc[2].tolist() == [2, 1, 0, -1]
    assert anc[5].tolist() == [5, 1, 0, -1]        # y_{0,1}: its anchor, then the trunk before it
    assert anc[6].tolist() == [6, 5, 1, 0]
    assert anc[7].tolist() == [7, 4, 3, 2]
    # the convolution reads exactly those rows: a one-hot input at row 4 reaches rows 4, 7 (tap 1)
    H, D, K = 1, 2, 4
    x = np.zeros((lay["n_rows"], H, D))
    x[4, 0, :] = 1.0
    w = np.zeros((H, D, K))
    w[0, :, 1] = 2.0
    y = conv_ancestry_ref(lay, x, w)
    hit = np.flatnonzero(np.abs(y[:, 0, 0]) > 0)
    assert hit.tolist() == [7]                      # row 4's only child is y_{1,1}
    assert np.isclose(y[7, 0, 0], silu(2.0))
    assert y[5, 0, 0] == 0.0                        # row 4 is not on y_{0,1}'s path


def test_step_closed_forms():
    g = np.random.default_rng(1)
    H, D = 3, 6
    S = g.standard_normal((H, D, D))
    q, v = g.standard_normal((H, D)), g.standard_normal((H, D))
    k = g.standard_normal((H, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    al = g.uniform(0.5, 1.0, H)
    be = g.uniform(0.1, 0.9, H)
    # no write: pure decay
    S1, o = gdn_step_ref(S, q, k, v, al, np.zeros(H))
    assert np.allclose(S1, al[:, None, None] * S, atol=1e-14)
    assert np.allclose(o, np.einsum("hvk,hk->hv", al[:, None, None] * S, q), atol=1e-13)
    # unit key, no decay: the read-out at k moves a fraction beta of the way to v
    S1, _ = gdn_step_ref(S, q, k, v, np.ones(H), be)
    want = (1 - be)[:, None] * np.einsum("hvk,hk->hv", S, k) + be[:, None] * v
    assert np.allclose(np.einsum("hvk,hk->hv", S1, k), want, atol=1e-13)
    # full write: the state reads back exactly v at k, whatever the decay
    S1, _ = gdn_step_ref(S, q, k, v, al, np.ones(H))
    assert np.allclose(np.einsum("hvk,hk->hv", S1, k), v, atol=1e-13)
    # basis key e_2, full write, no decay: only column 2 changes, and it becomes v
    e = np.zeros((H, D))
    e[:, 2] = 1.0
    S1, _ = gdn_step_ref(S, q, e, v, np.ones(H), np.ones(H))
    assert np.allclose(S1[:, :, 2], v, atol=1e-14)
    keep = [c for c in range(D) if c != 2]
    assert np.array_equal(S1[:, :, keep], S[:, :, keep])


def test_feature_norms_and_identity_taps():
    lay = pack_ref([9], [2], [3, 8], [4, 2])
    N, H, D = lay["n_rows"], 2, 8
    (xq, xk, xv), _, _, _ = _inputs(N, H, D, 1, 2)
    one = np.ones((H, D, 1))
    q, k, v = gdn_features_ref(lay, xq, xk, xv, one, one, one)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-14)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0 / np.sqrt(D), atol=1e-14)
    assert np.allclose(v, silu(xv), atol=1e-15)
    sk = silu(xk)
    assert np.allclose(k, sk / np.linalg.norm(sk, axis=-1, keepdims=True), atol=1e-14)


def _replay_vs_brute(lay, H, D, K, C, seed):
    N = lay["n_rows"]
    (xq, xk, xv), (wq, wk, wv), al, be = _inputs(N, H, D, K, seed)
    q, k, v = gdn_features_ref(lay, xq, xk, xv, wq, wk, wv)
    ck = gdn_checkpoints_ref(lay, q, k, v, al, be, C)
    ck0 = ck.copy()
    out = gdn_replay_ref(lay, q, k, v, al, be, ck, C)
    assert np.array_equal(ck, ck0)                              # checkpoints are read, never written
    worst = 0.0
    for b in range(lay["n_branches"]):
        W = int(lay["branch_len"][b])
        if W < 2:
            continue
        r0 = int(lay["branch_off"][b])
        want = gdn_branch_brute_ref(lay, xq, xk, xv, wq, wk, wv, al, be, b)
        worst = max(worst, float(np.abs(out[r0:r0 + W - 1] - want).max()))
    assert worst <= 1e-12, worst
    assert np.all(out[lay["row_branch"] < 0] == 0.0)            # trunk rows are not the replay's


@pytest.mark.parametrize("C,K", [(4, 4), (8, 4), (4, 1), (16, 2)])
def test_replay_equals_independent_scoring_edges(C, K):
    # anchors at 0, C-2, C-1, C, 2C-1, T-1, duplicates, and one-token branches
    T = 3 * C + 5
    anchors = [0, C - 2, C - 1, C, 2 * C - 1, T - 1, C - 1, 5]
    widths = [3, 4, 2, 5, 1, 6, 3, 1]
    lay = pack_ref([T], [len(anchors)], anchors, widths)
    _replay_vs_brute(lay, H=2, D=6, K=K, C=C, seed=C + K)


@pytest.mark.parametrize("seed", range(4))
def test_replay_equals_independent_scoring_random(seed):
    g = np.random.default_rng(100 + seed)
    nt = int(g.integers(1, 4))
    T = g.integers(1, 40, size=nt)
    nb = g.integers(0, 6, size=nt)
    anchors = np.concatenate([g.integers(0, T[t], size=nb[t]) for t in range(nt)]).astype(np.int32)
    widths = g.integers(1, 7, size=int(nb.sum())).astype(np.int32)
    lay = pack_ref(T.astype(np.int32), nb.astype(np.int32), anchors, widths)
    assert trunk_len_ref(lay).tolist() == T.tolist()
    _replay_vs_brute(lay, H=2, D=4, K=4, C=int(g.choice([4, 8])), seed=seed)


def test_branch_isolation_and_future_trunk():
    """A branch's outputs do not move when another branch's inputs or trunk tokens after its
    anchor change (checkpoints recomputed from the changed trunk)."""
    C, K, H, D = 4, 4, 2, 5
    T = 19
    lay = pack_ref([T], [3], [6, 13, 9], [4, 3, 5])
    N = lay["n_rows"]
    (xq, xk, xv), (wq, wk, wv), al, be = _inputs(N, H, D, K, 7)

    def run(xs):
        q, k, v = gdn_features_ref(lay, *xs, wq, wk, wv)
        ck = gdn_checkpoints_ref(lay, q, k, v, al, be, C)
        return gdn_replay_ref(lay, q, k, v, al, be, ck, C)

    base = run([xq, xk, xv])
    b = 0
    a, r0, W = int(lay["branch_anchor"][b]), int(lay["branch_off"][b]), int(lay["branch_len"][b])
    mine = np.arange(r0, r0 + W - 1)
    others = np.array([r for r in range(N) if r not in set(mine.tolist()) and not (r <= a)])
    g = np.random.default_rng(8)
    xs = [x.copy() for x in (xq, xk, xv)]
    for x in xs:
        x[others] = g.standard_normal(x[others].shape)
    moved = run(xs)
    assert np.array_equal(base[mine], moved[mine])


def test_trunk_outputs_equal_brute_sequence():
    """Trunk outputs against the brute-force scoring of a branch that copies the trunk:
    a branch anchored at trunk token 0 whose rows repeat the inputs of trunk tokens
    1 .. W-1 is the same sequence, so its outputs are the trunk's at those tokens."""
    C, K, H, D = 4, 4, 2, 5
    T, W = 13, 12
    lay = pack_ref([T], [1], [0], [W])
    N = lay["n_rows"]
    (xq, xk, xv), (wq, wk, wv), al, be = _inputs(N, H, D, K, 21)
    r0 = int(lay["branch_off"][0])
    for x in (xq, xk, xv, al, be):
        x[r0:r0 + W - 1] = x[1:W]
    q, k, v = gdn_features_ref(lay, xq, xk, xv, wq, wk, wv)
    ck, out = gdn_trunk_ref(lay, q, k, v, al, be, C)
    want = gdn_branch_brute_ref(lay, xq, xk, xv, wq, wk, wv, al, be, 0)
    assert np.abs(out[1:W] - want).max() <= 1e-12
    assert np.all(out[r0:] == 0.0)                                # branch rows are not the trunk's
    assert np.array_equal(ck, gdn_checkpoints_ref(lay, q, k, v, al, be, C))
    assert np.all(ck[0, 0] == 0.0)                                # slot 0: the zero state


@pytest.mark.parametrize("a,C", [(0, 4), (3, 4), (6, 4), (7, 8), (10, 4)])
def test_trunk_output_equals_replayed_copy(a, C):
    """A one-token-deeper branch at anchor a whose row copies trunk token a+1 has the
    ancestry, features and state of that token: the replay from checkpoints must give
    the trunk pass's output there (two routes: sequential vs checkpoint + replay)."""
    K, H, D = 3, 2, 6
    T = 12
    lay = pack_ref([T], [1], [a], [2])
    N = lay["n_rows"]
    (xq, xk, xv), (wq, wk, wv), al, be = _inputs(N, H, D, K, 30 + a)
    r0 = int(lay["branch_off"][0])
    for x in (xq, xk, xv, al, be):
        x[r0] = x[a + 1]
    q, k, v = gdn_features_ref(lay, xq, xk, xv, wq, wk, wv)
    ck, trunk = gdn_trunk_ref(lay, q, k, v, al, be, C)
    rep = gdn_replay_ref(lay, q, k, v, al, be, ck, C)
    assert np.abs(rep[r0] - trunk[a + 1]).max() <= 1e-13
