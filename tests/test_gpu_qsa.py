"""GPU parity: spec_qsa_attn_fwd (sparse attention with branch-consistent indexer groups)
against the float64 oracle."""
import numpy as np
import pytest

from _util import ATTN_ATOL, Case, from_device, say, to_device, widen
from oracle import tree_attn_ref
from oracle.qsa_ref import qsa_attn_ref, qsa_brute_force_branch_ref, qsa_group_keys, qsa_history_ref
from specgen import CONFIGS, gen_qsa_index, small_config

pytestmark = pytest.mark.gpu

PICK_RTOL = 1e-5   # float32 against float64 scores: picks may swap only inside this band


def _pack(s):
    import tree_attention_spec_amd as tas
    return tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])


def _run(case, idx, G, top_k, q=None, k=None, v=None, qi=None, ki=None):
    import torch
    import tree_attention_spec_amd as tas
    tree = _pack(case.s)
    if q is None:
        q, k, v = case.qkv()
    qi = idx["qi"] if qi is None else qi
    ki = idx["ki"] if ki is None else ki
    out, sel, ro = tas.spec_qsa_attn_fwd(tree, to_device(q), to_device(k), to_device(v), to_device(qi),
                                         to_device(ki), G, top_k, rope_base=case.cfg.rope_base)
    torch.cuda.synchronize()
    return out, sel, ro


def _exact_compare(case, G, top_k, grid=8, rows=None):
    """Grid-valued indexer inputs: every score is exact in float32, so the picks must be
    identical to the oracle's; outputs within the bf16 attention tolerance."""
    idx = gen_qsa_index(1, case.N, case.cfg.hkv, 32, grid=grid)
    out, sel, ro = _run(case, idx, G, top_k)
    q, k, v = case.qkv()
    want, picks = qsa_attn_ref(case.lay, widen(q), widen(k), widen(v), widen(idx["qi"]), widen(idx["ki"]), G,
                               top_k, case.cfg.rope_base, rows=rows)
    got = from_device(out) if rows is None else from_device(out)[rows]
    gsel = sel.cpu().numpy() if rows is None else sel.cpu().numpy()[rows]
    err = float(np.abs(got - want).max())
    say("  N=%d G=%d k=%d: max abs err %.3e, picks identical %s" % (case.N, G, top_k, err,
                                                                     np.array_equal(gsel, picks)))
    assert np.array_equal(gsel, picks)
    assert err <= ATTN_ATOL
    return out, sel, ro


@pytest.mark.parametrize("G,top_k", [(4, 2), (8, 3), (16, 1), (64, 2)])
def test_qsa_small_tree_exact_picks(G, top_k):
    say("qsa parity: small tree, grid indexer inputs")
    case = Case(small_config("stress", trunk=300, branches=14, width=16, hq=8, hkv=2, head_dim=128))
    _exact_compare(case, G, top_k)


def test_qsa_batched_trees_and_group_edges():
    """Two trees back to back; anchors at group edges (a = 0, G-1, G, 2G-1), duplicates and a
    one-token branch."""
    say("qsa parity: two trees, anchors at group edges")
    G = 8
    s = dict(trunk_len=np.array([90, 61], np.int32), n_branches=np.array([6, 3], np.int32),
             anchors=np.array([0, G - 1, G, 2 * G - 1, 2 * G - 1, 89, 5, 60, 31], np.int32),
             branch_len=np.array([9, 5, 1, 12, 3, 16, 7, 4, 10], np.int32))
    case = Case(small_config("batched", n_trees=2, hq=8, hkv=2, head_dim=128), structure=s)
    _exact_compare(case, G, 3)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 1), (12, 4)])
def test_qsa_head_groups(hq, hkv):
    """One query head per KV head, sixteen (every MFMA column used), and three."""
    say("qsa parity: %d query heads over %d KV heads" % (hq, hkv))
    case = Case(small_config("gqa8b", trunk=200, branches=8, width=9, hq=hq, hkv=hkv, head_dim=128))
    _exact_compare(case, 8, 4)


def test_qsa_branches_equal_their_own_sequences():
    """[SpecOPD notes page, "Checks, negative controls, and limits"]: every branch row of the
    packed result equals the oracle's scoring of that branch as its own sequence."""
    say("qsa: packed GPU result against each branch scored alone")
    G, top_k = 8, 3
    case = Case(small_config("stress", trunk=260, branches=10, width=16, hq=8, hkv=2, head_dim=128))
    idx = gen_qsa_index(2, case.N, case.cfg.hkv, 32, grid=8)
    out, sel, _ = _run(case, idx, G, top_k)
    got, gsel = from_device(out), sel.cpu().numpy()
    q, k, v = case.qkv()
    worst = 0.0
    for b in range(case.lay["n_branches"]):
        rows, ob, pb = qsa_brute_force_branch_ref(case.lay, widen(q), widen(k), widen(v), widen(idx["qi"]),
                                                  widen(idx["ki"]), b, G, top_k, case.cfg.rope_base)
        a = int(case.lay["branch_anchor"][b])
        mine = rows[a:]                          # the anchor row and the branch rows
        worst = max(worst, float(np.abs(got[mine] - ob[a:]).max()))
        assert np.array_equal(gsel[mine], pb[a:])
    say("  max abs err %.3e" % worst)
    assert worst <= ATTN_ATOL


def test_qsa_top_k_over_every_group_is_full_attention():
    say("qsa: top_k past the group count gives full tree attention")
    case = Case(small_config("gqa8b", trunk=150, branches=6, width=8, hq=8, hkv=2, head_dim=128))
    idx = gen_qsa_index(3, case.N, case.cfg.hkv, 16)
    out, sel, _ = _run(case, idx, 4, 64)
    q, k, v = case.qkv()
    want = tree_attn_ref(case.lay, widen(q), widen(k), widen(v), case.cfg.rope_base)
    err = float(np.abs(from_device(out) - want).max())
    say("  max abs err %.3e" % err)
    assert err <= ATTN_ATOL


def test_qsa_isolation_and_readout():
    """Changing every token outside a branch's history leaves its rows bit-identical; the
    readout is the predecessor row's output."""
    import torch
    say("qsa: isolation and readout")
    G, top_k = 8, 2
    case = Case(small_config("gqa8b", trunk=120, branches=6, width=8, hq=8, hkv=2, head_dim=128))
    idx = gen_qsa_index(4, case.N, case.cfg.hkv, 32)
    out1, sel1, ro = _run(case, idx, G, top_k)
    pr = torch.from_numpy(case.lay["step_pred_row"].astype(np.int64)).cuda()
    assert torch.equal(ro, out1[pr])
    q, k, v = case.qkv()
    rng = np.random.default_rng(9)
    for b in (0, 3, 5):
        mine = np.flatnonzero(case.lay["row_branch"] == b)
        keep = set(qsa_history_ref(case.lay, int(mine[-1])).tolist())
        other = np.array([r for r in range(case.N) if r not in keep])
        xs = [a.copy() for a in (q, k, v, idx["qi"], idx["ki"])]
        for a in xs:
            noise = rng.integers(0, 2 ** 15, size=a[other].shape).astype(np.uint16)
            a[other] = (noise & 0x3fff) | 0x3c00
        out2, sel2, _ = _run(case, idx, G, top_k, *xs)
        mt = torch.from_numpy(mine).cuda()
        assert torch.equal(out1[mt], out2[mt]) and torch.equal(sel1[mt], sel2[mt])


def _check_picks_valid(case, idx, rows, gsel, G, top_k, qd=None):
    """Normal-draw indexer inputs: where the GPU's float32 picks differ from the float64
    oracle's, every swapped group must score within PICK_RTOL of the k-th best score.
    Returns the rows whose picks equal the oracle's."""
    par = None
    from oracle import parents_ref
    par = parents_ref(case.lay)
    qi, ki = widen(idx["qi"]), widen(idx["ki"])
    same = []
    for n, r in enumerate(rows):
        hist = qsa_history_ref(case.lay, r, par)
        t = len(hist) - 1
        n_c = (t + 1) // G
        keys = qsa_group_keys(ki[hist[:n_c * G]], G)
        ok = True
        for g in range(case.cfg.hkv):
            sc = keys[:, g] @ qi[r, g]
            mine = gsel[n, g][gsel[n, g] >= 0]
            if n_c <= top_k:
                assert np.array_equal(mine, np.arange(n_c))
                continue
            kth = np.sort(sc)[::-1][top_k - 1]
            ref = np.sort(np.argsort(-sc, kind="stable")[:top_k])
            if not np.array_equal(mine, ref):
                ok = False
                diff = np.setxor1d(mine, ref)
                band = PICK_RTOL * max(abs(kth), 1e-30)
                assert np.all(np.abs(sc[diff] - kth) <= band), (r, g, sc[diff], kth)
        if ok:
            same.append(n)
    return np.array(same, dtype=np.int64)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["gqa8b", "stress"])
def test_qsa_workload_sampled(name):
    """Full-size tree in the benchmarked launch (G = 64, top_k = 16, index dim 64, N(0,1)
    indexer inputs): sampled rows' picks are valid top-k sets and, where they equal the
    oracle's, outputs match it."""
    from _util import sample_rows
    say("qsa parity: %s full size, sampled rows" % name)
    G, top_k, di = 64, 16, 64
    case = Case(CONFIGS[name])
    idx = gen_qsa_index(case.cfg.seed, case.N, case.cfg.hkv, di)
    out, sel, _ = _run(case, idx, G, top_k)
    rows = sample_rows(case.lay, 24)
    gsel = sel.cpu().numpy()[rows]
    same = _check_picks_valid(case, idx, rows, gsel, G, top_k)
    q, k, v = case.qkv()
    want, picks = qsa_attn_ref(case.lay, widen(q), widen(k), widen(v), widen(idx["qi"]), widen(idx["ki"]), G,
                               top_k, case.cfg.rope_base, rows=rows[same])
    err = float(np.abs(from_device(out[rows[same].tolist()]) - want).max())
    say("  %d rows, %d with the oracle's picks; max abs err %.3e" % (len(rows), len(same), err))
    assert len(same) >= 0.9 * len(rows)
    assert err <= ATTN_ATOL
