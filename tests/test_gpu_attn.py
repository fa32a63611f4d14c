"""GPU parity: spec_tree_attn_fwd (+ readout) against the float64 oracle."""
import numpy as np
import pytest

from _util import ATTN_ATOL, ATTN_ATOL_F32, Case, from_device, sample_rows, say, to_device, widen
from oracle import brute_force_branch_ref, readout_ref, tree_attn_ref
from specgen import CONFIGS, small_config

pytestmark = pytest.mark.gpu


def _run(case, q=None, k=None, v=None):
    import torch
    import tree_attention_spec_amd as tas
    s = case.s
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    if q is None:
        q, k, v = case.qkv()
    out, ro = tas.spec_tree_attn_fwd(tree, to_device(q), to_device(k), to_device(v),
                                     rope_base=case.cfg.rope_base)
    torch.cuda.synchronize()
    return out, ro


def _full_compare(case, atol):
    q, k, v = case.qkv()
    out, ro = _run(case)
    got = from_device(out)
    want = tree_attn_ref(case.lay, widen(q), widen(k), widen(v), case.cfg.rope_base)
    err = np.abs(got - want).max()
    say("  max abs err %.3e (N=%d)" % (err, case.N))
    assert err <= atol
    assert np.array_equal(from_device(ro), got[case.lay["step_pred_row"]])   # readout is a pure gather
    return got


def test_attn_tiny_f32():
    say("attn parity: tiny (fp32 path)")
    _full_compare(Case(CONFIGS["tiny"]), ATTN_ATOL_F32)


SMALL = [
    # several 64-key tiles, ragged tails, GQA groups 1/2/4/8, D 32/64/128, two trees
    dict(tag="s_d128_g4", base="gqa8b", trunk=300, branches=20, width=7, width_mode="uniform",
         hq=8, hkv=2, head_dim=128),
    dict(tag="s_d64_g1", base="gqa8b", trunk=197, branches=13, width=16, hq=4, hkv=4, head_dim=64),
    dict(tag="s_d32_g8", base="stress", trunk=150, branches=9, width=16, hq=16, hkv=2, head_dim=32,
         zipf_bias=None),
    dict(tag="s_2trees_g2", base="batched", n_trees=2, trunk=130, branches=11, width=8, hq=4, hkv=2,
         head_dim=128),
    dict(tag="s_d128_g8", base="stress", trunk=260, branches=30, width=16, hq=16, hkv=2, head_dim=128),
    # head dim 128 with GQA groups 1 and 3 (one and four waves per workgroup, a partial head slice)
    dict(tag="s_d128_g1", base="gqa8b", trunk=230, branches=12, width=9, hq=2, hkv=2, head_dim=128),
    dict(tag="s_d128_g3", base="gqa8b", n_trees=3, trunk=90, branches=5, width=11, hq=6, hkv=2, head_dim=128),
    # GQA group 16 (two workgroups of eight waves per block) and 5 (a partial second slice)
    dict(tag="s_d128_g16", base="stress", trunk=200, branches=9, width=16, hq=32, hkv=2, head_dim=128),
    dict(tag="s_d128_g5", base="gqa8b", trunk=170, branches=7, width=12, hq=10, hkv=2, head_dim=128),
]


@pytest.mark.parametrize("spec", SMALL, ids=[c["tag"] for c in SMALL])
def test_attn_small_bf16(spec):
    spec = dict(spec)
    base = spec.pop("base")
    say("attn parity: %s" % spec["tag"])
    _full_compare(Case(small_config(base, **spec)), ATTN_ATOL)


def test_attn_f32_general():
    say("attn parity: fp32 path, D=128 group 4")
    cfg = small_config("tiny", trunk=90, branches=7, width=9, width_mode="uniform", hq=8, hkv=2,
                       head_dim=128)
    _full_compare(Case(cfg), ATTN_ATOL_F32)


def test_attn_edge_trees():
    cfg = small_config("gqa8b", trunk=70, branches=0, hq=8, hkv=2, head_dim=128)
    cases = {
        "trunk only": dict(trunk_len=np.array([70]), n_branches=np.array([0]),
                           anchors=np.zeros(0, np.int32), branch_len=np.zeros(0, np.int32)),
        "anchors at 0 and T-1, one-token and duplicate": dict(
            trunk_len=np.array([70]), n_branches=np.array([6]),
            anchors=np.array([0, 69, 69, 5, 5, 33], np.int32),
            branch_len=np.array([16, 1, 40, 2, 2, 64], np.int32)),
        "single trunk row": dict(trunk_len=np.array([1]), n_branches=np.array([1]),
                                 anchors=np.array([0], np.int32), branch_len=np.array([3], np.int32)),
    }
    for tag, s in cases.items():
        say("attn parity: edge %s" % tag)
        _full_compare(Case(cfg, structure=s), ATTN_ATOL)


@pytest.mark.parametrize("head_dim", [128, 64])
def test_attn_moving_reference_and_scale(head_dim):
    """Scores that climb from key tile to key tile, with an explicit softmax scale.

    The query has a constant component 16 and each key the component 0.5 * (row // 16) in the
    slowest-turning RoPE pair (base 1e6, so that pair barely rotates): with scale 0.125 a query's
    largest visible score grows by ~6 log2 units per 64-key tile, so the online softmax moves its
    reference on most tiles. Trunk keys past a branch's anchor carry the largest scores of their
    tiles and must be masked before the maximum is taken.
    """
    from specgen import f32_to_bf16_bits
    say("attn parity: moving softmax reference, D=%d" % head_dim)
    cfg = small_config("gqa8b", trunk=333, branches=14, width=9, width_mode="uniform", hq=8, hkv=2,
                       head_dim=head_dim)
    case = Case(cfg)
    q, k, v = case.qkv()
    lay = case.lay
    j = head_dim // 2 - 1
    qf, kf = widen(q).astype(np.float32), widen(k).astype(np.float32)
    qf[:, :, j] = 16.0
    kf[:, :, j] = 0.5 * (np.arange(case.N) // 16)[:, None]
    q2, k2 = f32_to_bf16_bits(qf), f32_to_bf16_bits(kf)
    assert np.array_equal(widen(k2)[:, 0, j], kf[:, 0, j])          # the climbing component is exact
    import torch
    import tree_attention_spec_amd as tas
    s = case.s
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    out, ro = tas.spec_tree_attn_fwd(tree, to_device(q2), to_device(k2), to_device(v), rope_base=1e6,
                                     softmax_scale=0.125)
    torch.cuda.synchronize()
    got = from_device(out)
    want = tree_attn_ref(lay, widen(q2), widen(k2), widen(v), 1e6, scale=0.125)
    err = np.abs(got - want).max()
    say("  max abs err %.3e (N=%d)" % (err, case.N))
    assert np.isfinite(got).all()
    assert err <= ATTN_ATOL
    assert np.array_equal(from_device(ro), got[lay["step_pred_row"]])


def test_attn_isolation_is_bitwise():
    """Changing the values of every row outside a branch's history leaves its rows bit-identical."""
    import torch
    cfg = small_config("gqa8b", trunk=200, branches=12, width=16, hq=8, hkv=2, head_dim=128)
    case = Case(cfg)
    q, k, v = case.qkv()
    out1, _ = _run(case)
    lay = case.lay
    rng = np.random.default_rng(5)
    for b in [0, 5, 11]:
        mine = lay["row_branch"] == b
        keep = mine | ((lay["row_branch"] < 0) & (lay["row_pos"] <= lay["branch_anchor"][b]))
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        for a in (q2, k2, v2):
            noise = rng.integers(0, 2 ** 15, size=a[~keep].shape).astype(np.uint16)
            a[~keep] = (noise & 0x3fff) | 0x3c00   # other finite bf16 values
        out2, _ = _run(case, q2, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(out1[torch.from_numpy(mine).cuda()], out2[torch.from_numpy(mine).cuda()])


def test_attn_readout_leak():
    """Perturbing a sample's own row leaves its readout step bit-identical."""
    import torch
    cfg = small_config("gqa8b", trunk=100, branches=6, width=6, hq=8, hkv=2, head_dim=64)
    case = Case(cfg)
    q, k, v = case.qkv()
    _, ro1 = _run(case)
    lay = case.lay
    for s in range(0, lay["n_steps"], 5):
        srow = lay["step_sample_row"][s]
        if srow < 0:
            continue
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        for a in (q2, k2, v2):
            a[srow] ^= 0x0040
        _, ro2 = _run(case, q2, k2, v2)
        assert torch.equal(ro1[s], ro2[s])


@pytest.mark.slow
@pytest.mark.parametrize("name", ["gqa8b", "long", "batched", "stress"])
def test_attn_workload_sampled(name):
    """Full-size workloads in the benchmarked launch; sampled rows against the oracle."""
    say("attn parity: %s full size, sampled rows" % name)
    case = Case(CONFIGS[name])
    q, k, v = case.qkv()
    out, ro = _run(case)
    rows = sample_rows(case.lay, 40)
    got = from_device(out[rows.tolist()])
    want = tree_attn_ref(case.lay, widen(q), widen(k), widen(v), case.cfg.rope_base, rows=rows)
    err = np.abs(got - want).max()
    say("  %d rows, max abs err %.3e" % (len(rows), err))
    assert err <= ATTN_ATOL
    steps = np.arange(0, case.R, max(1, case.R // 64))
    import torch
    pr = torch.from_numpy(case.lay["step_pred_row"][steps].astype(np.int64)).cuda()
    assert torch.equal(ro[torch.from_numpy(steps).cuda()], out[pr])
    assert torch.isfinite(out.float()).all()


def test_attn_independent_layout_matches_oracle():
    """Every branch packed as its own tree (trunk through its anchor, then the branch): the
    uncached independent scoring the paper page's Figure 13 compares against. Every row of
    that layout equals the oracle's per-branch causal brute force, and its branch and anchor
    rows equal the shared-prefix layout's (same tokens, same positions)."""
    import torch
    import tree_attention_spec_amd as tas
    say("attn: independent per-branch layout vs the oracle's brute force and the shared prefix")
    case = Case(small_config("batched", n_trees=2, trunk=200, branches=9, width=8, hq=8, hkv=2,
                             head_dim=128))
    q, k, v = case.qkv()
    out, _ = _run(case)
    s, lay = case.s, case.lay
    a = s["anchors"].astype(np.int64)
    w = s["branch_len"].astype(np.int64)
    t_of_b = np.repeat(np.arange(len(s["trunk_len"])), s["n_branches"])
    trunk0 = lay["tree_off"][t_of_b].astype(np.int64)
    idx = np.concatenate([np.concatenate([trunk0[b] + np.arange(a[b] + 1), lay["branch_off"][b] + np.arange(w[b] - 1)])
                          for b in range(len(a))])
    tree_i = tas.spec_tree_pack((a + 1).astype(np.int32), np.ones(len(a), np.int32), a.astype(np.int32),
                                w.astype(np.int32))
    assert tree_i.n_rows == len(idx)
    out_i, _ = tas.spec_tree_attn_fwd(tree_i, to_device(q[idx]), to_device(k[idx]), to_device(v[idx]),
                                      rope_base=case.cfg.rope_base)
    torch.cuda.synchronize()
    oi = from_device(out_i)
    toff_i = from_device(tree_i.arrays()["tree_off"]).astype(np.int64)
    qd, kd, vd = widen(q), widen(k), widen(v)
    worst = 0.0
    for b in range(len(a)):
        rows_ref, o_ref = brute_force_branch_ref(lay, qd, kd, vd, b, case.cfg.rope_base)
        assert len(rows_ref) == a[b] + w[b]
        got = oi[toff_i[b]:toff_i[b] + a[b] + w[b]]
        worst = max(worst, float(np.abs(got - o_ref).max()))
    rows_s = np.concatenate([np.concatenate([[trunk0[b] + a[b]], lay["branch_off"][b] + np.arange(w[b] - 1)])
                             for b in range(len(a))])
    rows_i = np.concatenate([toff_i[b] + a[b] + np.arange(w[b]) for b in range(len(a))])
    diff = np.abs(from_device(out)[rows_s] - oi[rows_i]).max()
    say("  independent layout vs brute force: max abs err %.3e over %d rows; vs shared layout %.3e"
        % (worst, tree_i.n_rows, diff))
    assert worst <= ATTN_ATOL
    assert diff <= ATTN_ATOL
