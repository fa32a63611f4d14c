"""Pins for the head-formed E2E-TV oracle: the pages' teaching example read
through a head, exact one-hot readouts, the predecessor-row rule, the softmax
shift invariance and brute force on a tiny tree."""
import math

import numpy as np
import pytest

from oracle import e2etv_head_ref, e2etv_ref, head_logits_ref, pack_ref
from specgen import bf16_bits_to_f32, gen_head


def _log(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def _tiny_tree():
    # two trees' worth of branches in one: trunk 6, three branches of widths 1, 2, 3
    return pack_ref([6], [3], [0, 2, 5], [1, 2, 3])


def test_teaching_example_through_a_head(golden):
    g = golden("teaching_example.json")
    lay = pack_ref([1], [1], [0], [1])           # one branch of width 1 hung off row 0
    assert lay["step_pred_row"].tolist() == [0]  # the anchor row predicts the first sample
    p = np.asarray(g["teacher_probs"])
    head = np.stack([_log(p), np.zeros(3)], axis=1)   # column 0 holds log p
    hidden = np.array([[1.0, 0.0], [7.0, -3.0]])      # row 1 (the sample's own row) is not read
    z = _log(g["draft_probs"])[None]
    alpha, L, grad, _ = e2etv_head_ref(lay, hidden, head, z)
    assert alpha.tolist() == pytest.approx(g["alpha"], abs=1e-15)
    assert L == pytest.approx(g["loss"], abs=1e-15)
    assert grad[0, 2] == 0.0


def test_one_hot_readout_picks_head_columns():
    lay = _tiny_tree()
    N, R, V, d = lay["n_rows"], lay["n_steps"], 11, 5
    rng = np.random.default_rng(3)
    k_of_row = rng.integers(0, d, size=N)
    hidden = np.zeros((N, d))
    hidden[np.arange(N), k_of_row] = 1.0
    head = rng.normal(0, 2, size=(V, d))
    # teacher logits of step s are head column k(pred row of s), exactly
    y = head[:, k_of_row[lay["step_pred_row"]]].T
    assert np.array_equal(head_logits_ref(lay, hidden, head), y)
    z = rng.normal(0, 2, size=(R, V))
    want = e2etv_ref(z, y, lay["step_off"])
    got = e2etv_head_ref(lay, hidden, head, z)
    assert np.array_equal(got[0], want[0]) and got[1] == want[1]
    assert np.array_equal(got[2], want[2])


def test_only_predecessor_rows_are_read():
    lay = _tiny_tree()
    N, R, V, d = lay["n_rows"], lay["n_steps"], 9, 4
    rng = np.random.default_rng(4)
    hidden, head = rng.normal(size=(N, d)), rng.normal(size=(V, d))
    z = rng.normal(size=(R, V))
    a0 = e2etv_head_ref(lay, hidden, head, z)[0]
    pred = set(lay["step_pred_row"].tolist())
    for r in range(N):
        h2 = hidden.copy()
        h2[r] += 1.0
        a1 = e2etv_head_ref(lay, h2, head, z)[0]
        changed = set(np.flatnonzero(a1 != a0).tolist())
        want = set(np.flatnonzero(lay["step_pred_row"] == r).tolist())
        assert changed == want, (r, changed, want)
        assert (r in pred) == bool(want)
    # each branch's last sample has a row that no step reads
    last = lay["step_sample_row"][lay["step_off"][1:] - 1]
    assert not (set(last.tolist()) & pred)


def test_head_shift_leaves_alpha_unchanged():
    # adding one vector u to every head row shifts all logits of a row by h.u: softmax unchanged
    lay = _tiny_tree()
    N, R, V, d = lay["n_rows"], lay["n_steps"], 13, 6
    rng = np.random.default_rng(5)
    hidden, head = rng.normal(size=(N, d)), rng.normal(size=(V, d))
    z = rng.normal(size=(R, V))
    a0, L0, g0, _ = e2etv_head_ref(lay, hidden, head, z)
    a1, L1, g1, _ = e2etv_head_ref(lay, hidden, head + rng.normal(size=d), z)
    assert np.allclose(a1, a0, rtol=1e-12, atol=0) and L1 == pytest.approx(L0, abs=1e-12)
    assert np.allclose(g1, g0, rtol=0, atol=1e-12)
    # negative control: scaling one head row does change alpha
    h2 = head.copy()
    h2[0] *= 3.0
    assert not np.allclose(e2etv_head_ref(lay, hidden, h2, z)[0], a0)


def test_brute_force_tiny_bf16():
    lay = pack_ref([4], [2], [1, 3], [2, 1])
    N, R, V, d = lay["n_rows"], lay["n_steps"], 6, 3
    inp = gen_head(0, N, d, V, R)
    hidden = bf16_bits_to_f32(inp["hidden"]).astype(np.float64)
    head = bf16_bits_to_f32(inp["head"]).astype(np.float64)
    z = bf16_bits_to_f32(inp["draft"]).astype(np.float64)
    alpha, L, _, _ = e2etv_head_ref(lay, hidden, head, z)
    # plain loops: the branch of step s is read by walking the rows of the layout
    pred = lay["step_pred_row"].tolist()
    bf = []
    for s in range(R):
        y = [sum(hidden[pred[s]][k] * head[v][k] for k in range(d)) for v in range(V)]
        ey = [math.exp(t) for t in y]
        ez = [math.exp(t) for t in z[s]]
        bf.append(sum(min(a / sum(ez), b / sum(ey)) for a, b in zip(ez, ey)))
    assert alpha == pytest.approx(bf, rel=1e-12)
    off = lay["step_off"].tolist()
    tot = 0.0
    for b in range(len(off) - 1):
        pr = 1.0
        for s in range(off[b], off[b + 1]):
            pr *= bf[s]
            tot += pr
    assert L == pytest.approx(1 - tot / R, abs=1e-12)


def test_generator_scales():
    inp = gen_head(1, 8, 256, 64, 4)
    head = bf16_bits_to_f32(inp["head"]).astype(np.float64)
    assert inp["hidden"].shape == (8, 256) and head.shape == (64, 256) and inp["draft"].shape == (4, 64)
    assert 3.0 / 16 * 0.8 < head.std() < 3.0 / 16 * 1.2
