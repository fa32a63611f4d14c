"""Pins for the attention oracle: hand RoPE values, complex-rotation identity,
textbook causal attention (torch SDPA), brute-force branch scoring, closed forms,
isolation and the readout leak."""
import numpy as np
import pytest
import torch

from oracle import (brute_force_branch_ref, causal_attn_ref, pack_ref, readout_ref, rope_ref,
                    tree_attn_ref)


def _tree(rng, T=23, nb=5, wmax=5, hq=4, hkv=2, D=8, n_trees=1):
    Ts = [T] * n_trees
    nbs = [nb] * n_trees
    anchors = np.concatenate([rng.integers(0, T, size=nb) for _ in range(n_trees)])
    widths = rng.integers(1, wmax + 1, size=nb * n_trees)
    lay = pack_ref(Ts, nbs, anchors, widths)
    N = lay["n_rows"]
    q = rng.standard_normal((N, hq, D))
    k = rng.standard_normal((N, hkv, D))
    v = rng.standard_normal((N, hkv, D))
    return lay, q, k, v


def test_rope_hand_values(golden):
    g = golden("rope_example.json")
    for case in g["cases"]:
        got = rope_ref(np.array(case["x"]), case["pos"], g["base"])
        np.testing.assert_allclose(got, case["out"], rtol=0, atol=1e-15)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(1)
    D, base = 16, 500.0
    x = rng.standard_normal((5, D))
    pos = np.array([0, 1, 7, 123, 4095])
    half = D // 2
    z = x[:, :half] + 1j * x[:, half:]
    theta = np.exp(-np.log(base) * np.arange(0, D, 2) / D)      # base^(-2j/D) written via logs
    zr = z * np.exp(1j * pos[:, None] * theta)
    want = np.concatenate([zr.real, zr.imag], axis=1)
    np.testing.assert_allclose(rope_ref(x, pos, base), want, atol=1e-12)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(2)
    D = 32
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m, n, c in [(3, 1, 5), (100, 40, 999), (7, 7, 12345)]:
        a = rope_ref(q, m, 10000.0) @ rope_ref(k, n, 10000.0)
        b = rope_ref(q, m + c, 10000.0) @ rope_ref(k, n + c, 10000.0)
        assert abs(a - b) < 1e-10


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (8, 1)])
def test_causal_matches_torch_sdpa(hq, hkv):
    rng = np.random.default_rng(3)
    L, D, base = 19, 16, 10000.0
    q = rng.standard_normal((L, hq, D))
    k = rng.standard_normal((L, hkv, D))
    v = rng.standard_normal((L, hkv, D))
    got = causal_attn_ref(q, k, v, base)
    pos = np.arange(L)[:, None]
    qt = torch.from_numpy(rope_ref(q, pos, base)).permute(1, 0, 2)
    kt = torch.from_numpy(rope_ref(k, pos, base)).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    np.testing.assert_allclose(got, want.permute(1, 0, 2).numpy(), atol=1e-12)


def test_trunk_only_tree_is_causal():
    rng = np.random.default_rng(4)
    lay = pack_ref([17], [0], [], [])
    q, k, v = rng.standard_normal((17, 4, 8)), rng.standard_normal((17, 2, 8)), rng.standard_normal((17, 2, 8))
    np.testing.assert_allclose(tree_attn_ref(lay, q, k, v, 10000.0), causal_attn_ref(q, k, v, 10000.0),
                               atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_packed_equals_brute_force(seed):
    rng = np.random.default_rng(10 + seed)
    lay, q, k, v = _tree(rng, n_trees=1 + seed % 2)
    o = tree_attn_ref(lay, q, k, v, 10000.0)
    for b in range(lay["n_branches"]):
        rows, ob = brute_force_branch_ref(lay, q, k, v, b, 10000.0)
        np.testing.assert_allclose(o[rows], ob, atol=1e-12, rtol=0)


def test_zero_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(5)
    lay, q, k, v = _tree(rng)
    o = tree_attn_ref(lay, q, np.zeros_like(k), v, 10000.0)
    for r in range(lay["n_rows"]):
        t = lay["row_tree"][r]
        vis = list(range(lay["tree_off"][t], lay["row_trunk_hi"][r] + 1)) + list(range(lay["row_branch_lo"][r], r + 1))
        want = v[vis].mean(axis=0).repeat(2, axis=0)      # Hq/Hkv = 2 heads share a KV head
        np.testing.assert_allclose(o[r], want, atol=1e-12)


def test_constant_values_give_the_constant():
    rng = np.random.default_rng(6)
    lay, q, k, v = _tree(rng)
    o = tree_attn_ref(lay, q, k, np.full_like(v, 0.375), 10000.0)
    np.testing.assert_allclose(o, 0.375, atol=1e-13)


def test_isolation_from_siblings_and_future():
    rng = np.random.default_rng(7)
    lay, q, k, v = _tree(rng, T=30, nb=6, wmax=6)
    o = tree_attn_ref(lay, q, k, v, 10000.0)
    for b in range(lay["n_branches"]):
        mine = lay["row_branch"] == b
        if not mine.any():
            continue
        a = lay["branch_anchor"][b]
        # change every row that is neither in branch b nor in the trunk prefix through a_b
        other = ~mine & ~((lay["row_branch"] < 0) & (lay["row_pos"] <= a))
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[other] += 3.0
        k2[other] -= 2.0
        v2[other] *= -5.0
        o2 = tree_attn_ref(lay, q2, k2, v2, 10000.0)
        assert np.array_equal(o2[mine], o[mine])


def test_readout_never_reads_own_row():
    rng = np.random.default_rng(8)
    lay, q, k, v = _tree(rng, T=20, nb=5, wmax=5)
    ro = readout_ref(lay, tree_attn_ref(lay, q, k, v, 10000.0))
    for s in range(lay["n_steps"]):
        srow = lay["step_sample_row"][s]
        if srow < 0:
            continue
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[srow] += 1.0
        k2[srow] += 1.0
        v2[srow] += 1.0
        ro2 = readout_ref(lay, tree_attn_ref(lay, q2, k2, v2, 10000.0))
        assert np.array_equal(ro2[s], ro[s])                 # the sample's own row never feeds its step
        p = lay["step_pred_row"][s]
        q3 = q.copy()
        q3[p] += 1.0
        ro3 = readout_ref(lay, tree_attn_ref(lay, q3, k, v, 10000.0))
        assert not np.array_equal(ro3[s], ro[s])             # its predecessor row does


def test_readout_feeds_a_head_end_to_end():
    """Readout rows through a random head give logits whose step order follows the pack."""
    rng = np.random.default_rng(9)
    lay, q, k, v = _tree(rng, T=16, nb=4, wmax=4)
    o = tree_attn_ref(lay, q, k, v, 10000.0)
    head = rng.standard_normal((o.shape[1] * o.shape[2], 11))
    logits = readout_ref(lay, o).reshape(lay["n_steps"], -1) @ head
    for s in range(lay["n_steps"]):
        np.testing.assert_allclose(logits[s], o[lay["step_pred_row"][s]].reshape(-1) @ head, atol=1e-12)
