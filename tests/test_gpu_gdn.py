"""GPU parity: spec_gdn_replay_fwd against the float64 oracle (indexed replay from
the same float32 checkpoints), plus each branch scored as its own sequence;
spec_gdn_trunk_fwd's outputs and checkpoints against the oracle's trunk pass, and
the two entry points chained (trunk pass, then replay from its checkpoints)."""
import numpy as np
import pytest

from _util import say, to_device, widen
from oracle import (gdn_branch_brute_ref, gdn_checkpoints_ref, gdn_features_ref, gdn_replay_ref,
                    gdn_trunk_ref, pack_ref)
from specgen import CONFIGS, gen_gdn, gen_gdn_states, gen_structure

pytestmark = pytest.mark.gpu

# float32 state and features against float64, relative to the largest output: the
# recurrence's rounding over at most C - 1 + W - 1 steps of D-term float32 sums gives
# ~1e-6 (measured <= 4e-7 on the small cases)
GDN_RTOL = 1e-5


def _run(s, lay, H, D, K, C, ckpt_kmajor, inp):
    import torch
    import tree_attention_spec_amd as tas
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    assert tree.max_trunk_len == int(np.max(s["trunk_len"]))
    dev = lambda a: to_device(np.ascontiguousarray(a))
    out = torch.full((lay["n_rows"], H, D), 7.0, dtype=torch.float32, device="cuda")
    tas.spec_gdn_replay_fwd(tree, dev(inp["xq"]), dev(inp["xk"]), dev(inp["xv"]), dev(inp["taps"]),
                            dev(inp["alpha"]), dev(inp["beta"]), dev(ckpt_kmajor), chunk=C, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _features(lay, inp):
    t = inp["taps"].astype(np.float64)
    return gdn_features_ref(lay, widen(inp["xq"]), widen(inp["xk"]), widen(inp["xv"]), t[0], t[1], t[2])


def _compare(s, H, D, K, C, seed, brute=True):
    lay = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    inp = gen_gdn(seed, lay["n_rows"], H, D, K)
    q, k, v = _features(lay, inp)
    al, be = inp["alpha"].astype(np.float64), inp["beta"].astype(np.float64)
    ck = gdn_checkpoints_ref(lay, q, k, v, al, be, C).astype(np.float32)      # the trunk pass's states
    got = _run(s, lay, H, D, K, C, np.swapaxes(ck, -1, -2), inp)
    want = gdn_replay_ref(lay, q, k, v, al, be, ck.astype(np.float64), C)
    br = lay["row_branch"] >= 0
    scale = max(np.abs(want[br]).max(), 1e-30) if br.any() else 1.0
    err = np.abs(got[br] - want[br]).max() if br.any() else 0.0
    say("  N=%d H=%d D=%d K=%d C=%d: max abs err %.3e (max |o| %.3e)" % (lay["n_rows"], H, D, K, C, err, scale))
    assert err <= GDN_RTOL * scale
    assert np.all(got[~br] == 7.0)                                              # trunk rows untouched
    if brute:   # the GPU against each branch as its own sequence (no checkpoints, no parent array)
        t = inp["taps"].astype(np.float64)
        for b in range(lay["n_branches"]):
            W = int(lay["branch_len"][b])
            if W < 2:
                continue
            r0 = int(lay["branch_off"][b])
            ref = gdn_branch_brute_ref(lay, widen(inp["xq"]), widen(inp["xk"]), widen(inp["xv"]),
                                       t[0], t[1], t[2], al, be, b)
            # the checkpoints went through float32, so allow their rounding too
            assert np.abs(got[r0:r0 + W - 1] - ref).max() <= 2 * GDN_RTOL * scale


CASES = [
    # (tag, trunk lengths, anchors per tree, widths, H, D, K, C)
    ("d128_k4_c64", [200], [[0, 62, 63, 64, 127, 199, 63, 17]], [[5, 3, 9, 2, 1, 16, 4, 7]], 2, 128, 4, 64),
    ("d64_k4_c16", [90], [[0, 15, 16, 47, 89, 30, 30]], [[3, 6, 2, 1, 9, 4, 4]], 3, 64, 4, 16),
    ("d128_k1_c8", [41], [[0, 7, 8, 40, 21]], [[4, 2, 6, 3, 1]], 1, 128, 1, 8),
    ("d64_k2_c4_2trees", [23, 9], [[0, 3, 4, 22, 11], [8, 0, 5]], [[2, 5, 3, 6, 1], [4, 3, 2]], 2, 64, 2, 4),
    ("d128_k3_c64_shortT", [30, 70], [[29, 0, 10], [69, 63, 64]], [[6, 3, 2], [4, 5, 8]], 1, 128, 3, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gdn_small(case):
    tag, T, anchors, widths, H, D, K, C = case
    say("gdn parity: %s" % tag)
    s = dict(trunk_len=np.array(T, np.int32), n_branches=np.array([len(a) for a in anchors], np.int32),
             anchors=np.concatenate([np.array(a, np.int32) for a in anchors]),
             branch_len=np.concatenate([np.array(w, np.int32) for w in widths]))
    _compare(s, H, D, K, C, seed=len(tag))


def test_gdn_no_branch_rows():
    """Only one-token branches (no rows): nothing is written."""
    say("gdn parity: one-token branches only")
    s = dict(trunk_len=np.array([50], np.int32), n_branches=np.array([3], np.int32),
             anchors=np.array([0, 20, 49], np.int32), branch_len=np.array([1, 1, 1], np.int32))
    _compare(s, 2, 64, 4, 16, seed=3, brute=False)


@pytest.mark.slow
def test_gdn_workload_sampled():
    """The 8B-like tree (trunk 4096, 256 branches of width 16) with 32 heads of 128, width-4
    convolution and checkpoints every 64 tokens, in the benchmarked launch; stand-in
    checkpoint states; sampled branches against the oracle."""
    import torch
    import tree_attention_spec_amd as tas
    cfg = CONFIGS["gqa8b"]
    s = gen_structure(cfg)
    lay = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    H, D, K, C = 32, 128, 4, 64
    say("gdn parity: 8B-like tree full size, sampled branches")
    inp = gen_gdn(cfg.seed, lay["n_rows"], H, D, K)
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    slots = tas.gdn_checkpoint_slots(tree, C)
    st = gen_gdn_states(cfg.seed, slots, H, D)[None]                            # [1, slots, H, D, D]
    got = _run(s, lay, H, D, K, C, st, inp)
    q, k, v = _features(lay, inp)
    al, be = inp["alpha"].astype(np.float64), inp["beta"].astype(np.float64)
    pick = np.random.default_rng(0).choice(lay["n_branches"], size=8, replace=False).tolist()
    pick += [int(np.argmax(lay["branch_anchor"])), int(np.argmin(lay["branch_anchor"]))]
    want = gdn_replay_ref(lay, q, k, v, al, be, np.swapaxes(st, -1, -2).astype(np.float64), C,
                          branches=pick)
    for b in pick:
        r0, W = int(lay["branch_off"][b]), int(lay["branch_len"][b])
        rows = slice(r0, r0 + W - 1)
        scale = np.abs(want[rows]).max()
        err = np.abs(got[rows] - want[rows]).max()
        assert err <= GDN_RTOL * scale, (b, err, scale)
    say("  sampled %d branches ok" % len(pick))
    torch.cuda.synchronize()


def _trunk_compare(s, H, D, K, C, seed, heads=None):
    """Trunk pass then replay on the GPU; the oracle's trunk pass and replay in float64
    (on the given subset of heads, default all)."""
    import torch
    import tree_attention_spec_amd as tas
    lay = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    inp = gen_gdn(seed, lay["n_rows"], H, D, K)
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    dev = lambda a: to_device(np.ascontiguousarray(a))
    x = [dev(inp[n]) for n in ("xq", "xk", "xv", "taps", "alpha", "beta")]
    slots = tas.gdn_checkpoint_slots(tree, C)
    ck_g = torch.full((lay["n_trees"], slots, H, D, D), 5.0, dtype=torch.float32, device="cuda")
    out_g = torch.full((lay["n_rows"], H, D), 7.0, dtype=torch.float32, device="cuda")
    work = torch.empty(tas.gdn_trunk_work_bytes(tree, H, D, K, C), dtype=torch.uint8, device="cuda")
    tas.spec_gdn_trunk_fwd(tree, *x, chunk=C, ckpt=ck_g, out=out_g, work=work)
    trunk_out = out_g.clone()
    tas.spec_gdn_replay_fwd(tree, *x, ckpt=ck_g, chunk=C, out=out_g)              # token at a time
    outs = [out_g]
    if C <= 64:                                                                 # from the trunk cache
        out_c = trunk_out.clone()
        tas.spec_gdn_replay_fwd(tree, *x, ckpt=ck_g, chunk=C, out=out_c, trunk_work=work)
        outs.append(out_c)
    torch.cuda.synchronize()
    hs = list(range(H)) if heads is None else list(heads)
    tr = lay["row_branch"] < 0
    T = np.asarray(s["trunk_len"])
    # whole-tensor checks on the device: branch rows untouched by the trunk pass, slots a
    # tree never reaches untouched, slot 0 the zero state, the replays leave trunk rows
    trg = torch.from_numpy(tr).cuda()
    assert bool((trunk_out[~trg] == 7.0).all())
    for ti in range(lay["n_trees"]):
        reach = int(T[ti]) // C + 1
        assert bool((ck_g[ti, 0] == 0.0).all()) and bool((ck_g[ti, reach:] == 5.0).all())
    for o in outs:
        assert torch.equal(o[trg], trunk_out[trg])
    hsg = torch.tensor(hs, device="cuda")
    ck = np.swapaxes(ck_g.index_select(2, hsg).cpu().numpy().astype(np.float64), -1, -2)  # value-major
    trunk_got = trunk_out.index_select(1, hsg).cpu().numpy().astype(np.float64)

    sub = lambda a: np.ascontiguousarray(a[:, hs])
    t = inp["taps"].astype(np.float64)[:, hs]
    q, k, v = gdn_features_ref(lay, sub(widen(inp["xq"])), sub(widen(inp["xk"])), sub(widen(inp["xv"])),
                               t[0], t[1], t[2])
    al, be = sub(inp["alpha"].astype(np.float64)), sub(inp["beta"].astype(np.float64))
    ck_ref, o_ref = gdn_trunk_ref(lay, q, k, v, al, be, C)
    # trunk outputs
    scale = np.abs(o_ref[tr]).max()
    err = np.abs(trunk_got[tr] - o_ref[tr]).max()
    say("  trunk outputs: max abs err %.3e (max |o| %.3e)" % (err, scale))
    assert err <= GDN_RTOL * scale
    # checkpoints: every slot a tree reaches
    for ti in range(lay["n_trees"]):
        reach = int(T[ti]) // C + 1
        cs = np.abs(ck_ref[ti, :reach]).max() if reach > 1 else 1.0
        cerr = np.abs(ck[ti, :reach] - ck_ref[ti, :reach]).max()
        say("  tree %d: %d checkpoints, max abs err %.3e (max |S| %.3e)" % (ti, reach, cerr, cs))
        assert cerr <= GDN_RTOL * cs
    # both replays from the GPU's checkpoints against the oracle's chained path
    br = lay["row_branch"] >= 0
    if br.any():
        want = gdn_replay_ref(lay, q, k, v, al, be, ck_ref, C)
        for name, o in zip(("token-at-a-time", "cached"), outs):
            got = o.index_select(1, hsg).cpu().numpy().astype(np.float64)
            bs = np.abs(want[br]).max()
            berr = np.abs(got[br] - want[br]).max()
            say("  %s replay: max abs err %.3e (max |o| %.3e)" % (name, berr, bs))
            assert berr <= 2 * GDN_RTOL * bs


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gdn_trunk_small(case):
    tag, T, anchors, widths, H, D, K, C = case
    say("gdn trunk pass: %s" % tag)
    s = dict(trunk_len=np.array(T, np.int32), n_branches=np.array([len(a) for a in anchors], np.int32),
             anchors=np.concatenate([np.array(a, np.int32) for a in anchors]),
             branch_len=np.concatenate([np.array(w, np.int32) for w in widths]))
    _trunk_compare(s, H, D, K, C, seed=len(tag) + 50)


def test_gdn_trunk_edges():
    """Trunks of one token, of exactly C and of C - 1 tokens, and a tree with no branches."""
    say("gdn trunk pass: edge trunk lengths")
    s = dict(trunk_len=np.array([1, 16, 15, 33], np.int32), n_branches=np.array([1, 2, 0, 1], np.int32),
             anchors=np.array([0, 15, 3, 32], np.int32), branch_len=np.array([3, 2, 4, 5], np.int32))
    _trunk_compare(s, 2, 64, 4, 16, seed=77)


CACHE_CASES = [
    # (tag, trunk lengths, anchors, widths, H, D, K, C): widths past 17 and 33 take the 32- and
    # 64-row branch tiles; anchors at cC - 1 (nothing to replay), cC (one token), cC + C - 2
    # (63 tokens) and in a last partial chunk
    ("w20_d128", [200], [63, 64, 126, 190, 5], [20, 18, 3, 20, 1], 2, 128, 4, 64),
    ("w40_d64", [150], [0, 63, 127, 149, 100], [40, 34, 2, 40, 33], 2, 64, 3, 64),
    ("w64_d128", [130], [64, 129, 10], [64, 64, 17], 1, 128, 2, 64),
    ("c16_two_trees", [40, 70], [15, 16, 39, 0, 47, 69], [9, 5, 16, 2, 12, 7], 2, 64, 4, 16),
]


@pytest.mark.parametrize("case", CACHE_CASES, ids=[c[0] for c in CACHE_CASES])
def test_gdn_replay_from_trunk_cache(case):
    tag, T, anchors, widths, H, D, K, C = case
    say("gdn replay from the trunk cache: %s" % tag)
    nb = [len(anchors)] if len(T) == 1 else [3, 3]
    s = dict(trunk_len=np.array(T, np.int32), n_branches=np.array(nb, np.int32),
             anchors=np.array(anchors, np.int32), branch_len=np.array(widths, np.int32))
    _trunk_compare(s, H, D, K, C, seed=len(tag) + 7)


def test_gdn_trunk_token_at_a_time():
    """Checkpoints every 128 tokens take the token-at-a-time trunk pass."""
    say("gdn trunk pass: chunk 128 (token at a time)")
    s = dict(trunk_len=np.array([300, 128], np.int32), n_branches=np.array([3, 1], np.int32),
             anchors=np.array([127, 128, 299, 127], np.int32), branch_len=np.array([4, 3, 5, 2], np.int32))
    _trunk_compare(s, 2, 128, 4, 128, seed=91)


def test_gdn_trunk_work_reuse():
    """One workspace and checkpoint buffer reused for two trees in a row (the second
    smaller) gives the same results as fresh buffers."""
    import torch
    import tree_attention_spec_amd as tas
    say("gdn trunk pass: workspace reuse")
    H, D, K, C = 2, 64, 4, 16
    outs = []
    work = None
    for T in ([150, 40], [33]):
        s = dict(trunk_len=np.array(T, np.int32), n_branches=np.zeros(len(T), np.int32),
                 anchors=np.zeros(0, np.int32), branch_len=np.zeros(0, np.int32))
        tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
        inp = gen_gdn(5, tree.n_rows, H, D, K)
        x = [to_device(np.ascontiguousarray(inp[n])) for n in ("xq", "xk", "xv", "taps", "alpha", "beta")]
        if work is None:
            work = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        ck1, o1 = tas.spec_gdn_trunk_fwd(tree, *x, chunk=C, work=work)
        ck2, o2 = tas.spec_gdn_trunk_fwd(tree, *x, chunk=C)
        torch.cuda.synchronize()
        assert torch.equal(ck1, ck2) and torch.equal(o1, o2)
        outs.append(o1)
    say("  bit-identical with a reused workspace")


@pytest.mark.slow
def test_gdn_trunk_workload_sampled_heads():
    """The 8B-like tree with 32 heads of 128, width-4 convolution, checkpoints every 64
    tokens: the whole trunk pass and replay on the GPU, 3 heads against the oracle."""
    cfg = CONFIGS["gqa8b"]
    say("gdn trunk pass + replay: 8B-like tree full size, heads 0, 17, 31")
    _trunk_compare(gen_structure(cfg), 32, 128, 4, 64, seed=cfg.seed, heads=[0, 17, 31])


@pytest.mark.slow
@pytest.mark.parametrize("name", ["long", "batched", "stress"])
def test_gdn_other_workloads_sampled_heads(name):
    """The other workloads' trees at full size (a 16,384-token trunk; 8 trees of 2,048;
    a 32,768-token trunk with widths 1..16 and 64 heads), trunk pass and both replays on
    the GPU for all heads, two heads against the oracle."""
    cfg = CONFIGS[name]
    say("gdn trunk pass + replay: %s tree full size, %d heads, heads 1 and last" % (name, cfg.hq))
    _trunk_compare(gen_structure(cfg), cfg.hq, 128, 4, 64, seed=cfg.seed, heads=[1, cfg.hq - 1])
