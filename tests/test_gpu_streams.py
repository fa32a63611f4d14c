"""Every entry point enqueues its work on the caller's stream: the whole path run on a
side stream gives results bit-identical to the default stream, and a reused
workspace gives the same results as a fresh one."""
import numpy as np
import pytest

from _util import say, to_device
from specgen import gen_gdn, gen_gdn_states, gen_logits, gen_qkv, gen_structure, small_config

pytestmark = pytest.mark.gpu


def _inputs():
    cfg = small_config("gqa8b", trunk=300, branches=14, width=9, width_mode="uniform", hq=8, hkv=2,
                       vocab=8192)
    s = gen_structure(cfg)
    import tree_attention_spec_amd as tas
    lay, _ = tas.spec_tree_pack_query(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    q, k, v = gen_qkv(cfg, lay.n_rows)
    z, y = gen_logits(cfg, lay.n_steps)
    g = gen_gdn(2, lay.n_rows, 2, 128, 4)
    slots = lay.max_trunk_len // 16 + 1
    st = gen_gdn_states(2, slots, 2, 128).reshape(1, slots, 2, 128, 128)
    return cfg, s, dict(q=q, k=k, v=v, z=z, y=y), g, st


def _path(cfg, s, d, g, st, awork=None, ework=None):
    import torch
    import tree_attention_spec_amd as tas
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    out, ro = tas.spec_tree_attn_fwd(tree, d["q"], d["k"], d["v"], rope_base=cfg.rope_base, work=awork)
    alpha, loss, grad = tas.spec_e2etv_fwd_bwd(tree, d["z"], d["y"], work=ework)
    o_gdn = tas.spec_gdn_replay_fwd(tree, g["xq"], g["xk"], g["xv"], g["taps"], g["alpha"], g["beta"],
                                    st, chunk=16)
    return [out, ro, alpha, loss, grad, o_gdn]


def test_side_stream_and_workspace_reuse():
    import torch
    import tree_attention_spec_amd as tas
    say("streams: the path on the default stream, on a side stream, and with reused workspaces")
    cfg, s, host, gh, sth = _inputs()
    d = {k: to_device(v) for k, v in host.items()}
    g = {k: to_device(v) for k, v in gh.items()}
    st = to_device(sth)
    ref = _path(cfg, s, d, g, st)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = _path(cfg, s, d, g, st)
    side.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    # one pair of workspaces serving two calls in a row
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    awork = torch.empty(tas.attn_work_bytes(tree, cfg.hq, cfg.hkv, cfg.head_dim, d["q"].dtype),
                        dtype=torch.uint8, device="cuda")
    ework = torch.empty(tas.e2etv_work_bytes(tree, cfg.vocab, d["z"].dtype), dtype=torch.uint8,
                        device="cuda")
    for _ in range(2):
        got = _path(cfg, s, d, g, st, awork=awork, ework=ework)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    say("  %d outputs identical on the side stream and with reused workspaces" % len(ref))
