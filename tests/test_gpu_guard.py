"""GPU: every entry point writes its outputs and nothing next to them.

Each output tensor is a view into a larger buffer whose guard bands before and after
it hold a sentinel bit pattern; after the call the bands must be unchanged. Covers the
tiled (head dim 128) and register-staged (64) bf16 attention, the float32 attention,
the fused and fallback E2E-TV paths, the allocation-free E2E-TV, the fused LM head and
sparse attention."""
import numpy as np
import pytest

from _util import Case, say, to_device
from specgen import gen_head, gen_qsa_index, small_config

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements on each side (a multiple of 16 bytes for every dtype here)


def _guarded(shape, dtype):
    """(buffer, view): the view has `shape`; the buffer's bands hold a sentinel."""
    import torch
    n = int(np.prod(shape))
    if dtype == torch.bfloat16:
        buf = torch.empty(n + 2 * GUARD, dtype=torch.int16, device="cuda").fill_(0x7FB5).view(torch.bfloat16)
    elif dtype == torch.float32:
        buf = torch.empty(n + 2 * GUARD, dtype=torch.int32, device="cuda").fill_(0x7FB5A5A5).view(torch.float32)
    else:
        buf = torch.full((n + 2 * GUARD,), -0x5A5A5A5B, dtype=dtype, device="cuda")
    ref = buf.clone()
    return (buf, ref), buf[GUARD:GUARD + n].view(*shape)


def _check(name, guarded):
    import torch
    buf, ref = guarded
    torch.cuda.synchronize()
    bands = lambda t: (t[:GUARD].view(torch.uint8), t[-GUARD:].view(torch.uint8))
    (b0, b1), (r0, r1) = bands(buf), bands(ref)
    ok = torch.equal(b0, r0) and torch.equal(b1, r1)
    say("  %s: guard bands %s" % (name, "intact" if ok else "WRITTEN"))
    assert ok, name


def _pack(case):
    import tree_attention_spec_amd as tas
    s = case.s
    return tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])


@pytest.mark.parametrize("head_dim,dtype", [(128, "bf16"), (64, "bf16"), (64, "f32")])
def test_attention_outputs_guarded(head_dim, dtype):
    import torch
    import tree_attention_spec_amd as tas
    say("guard bands: attention, head dim %d, %s" % (head_dim, dtype))
    case = Case(small_config("gqa8b", trunk=300, branches=11, width=9, hq=8, hkv=2, head_dim=head_dim,
                             qkv_dtype=dtype))
    tree = _pack(case)
    q, k, v = (to_device(a) for a in case.qkv())
    g_out, out = _guarded(tuple(q.shape), q.dtype)
    g_ro, ro = _guarded((tree.n_steps, q.shape[1], head_dim), q.dtype)
    tas.spec_tree_attn_fwd(tree, q, k, v, rope_base=case.cfg.rope_base, out=out, readout_out=ro)
    _check("out", g_out)
    _check("readout", g_ro)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("logit_dtype,vocab", [("bf16", 4104), ("f32", 1000)])
def test_e2etv_outputs_guarded(logit_dtype, vocab):
    import torch
    import tree_attention_spec_amd as tas
    say("guard bands: E2E-TV, %s logits, V %d" % (logit_dtype, vocab))
    case = Case(small_config("stress", trunk=400, branches=20, width=16, vocab=vocab, logit_dtype=logit_dtype))
    tree = _pack(case)
    z, y = (to_device(a) for a in case.logits())
    R = tree.n_steps
    g_a, alpha = _guarded((R,), torch.float32)
    g_l, loss = _guarded((1,), torch.float32)
    g_g, grad = _guarded((R, vocab), torch.float32)
    tas.spec_e2etv_fwd_bwd(tree, z, y, alpha_out=alpha, loss_out=loss, grad_out=grad)
    for name, gb in (("alpha", g_a), ("loss", g_l), ("grad", g_g)):
        _check(name, gb)
    if logit_dtype == "bf16":
        g_a2, alpha2 = _guarded((R,), torch.float32)
        g_l2, loss2 = _guarded((1,), torch.float32)
        g_g2, grad2 = _guarded((R, vocab), torch.float32)
        tas.spec_e2etv_fwd_bwd_noalloc(tree, z, y, alpha_out=alpha2, loss_out=loss2, grad_out=grad2)
        for name, gb in (("alpha (no-alloc)", g_a2), ("loss (no-alloc)", g_l2), ("grad (no-alloc)", g_g2)):
            _check(name, gb)
        assert torch.equal(alpha, alpha2) and torch.equal(grad, grad2)


def test_head_outputs_guarded():
    import torch
    import tree_attention_spec_amd as tas
    say("guard bands: E2E-TV through the output head")
    case = Case(small_config("stress", trunk=500, branches=40, width=16, vocab=1000))
    tree = _pack(case)
    d, V = 128, 1000
    inp = gen_head(0, case.N, d, V, case.R, 3.0)
    draft, hidden, head = (to_device(inp[k]) for k in ("draft", "hidden", "head"))
    R = tree.n_steps
    g_a, alpha = _guarded((R,), torch.float32)
    g_l, loss = _guarded((1,), torch.float32)
    g_g, grad = _guarded((R, V), torch.float32)
    tas.spec_e2etv_head_fwd_bwd(tree, draft, hidden, head, alpha_out=alpha, loss_out=loss, grad_out=grad)
    for name, gb in (("alpha", g_a), ("loss", g_l), ("grad", g_g)):
        _check(name, gb)


def test_qsa_outputs_guarded():
    import torch
    import tree_attention_spec_amd as tas
    say("guard bands: sparse attention")
    case = Case(small_config("gqa8b", trunk=200, branches=8, width=9, hq=8, hkv=2, head_dim=128))
    tree = _pack(case)
    idx = gen_qsa_index(1, case.N, case.cfg.hkv, 32)
    q, k, v = (to_device(a) for a in case.qkv())
    G, top_k = 8, 3
    g_out, out = _guarded(tuple(q.shape), q.dtype)
    g_sel, sel = _guarded((case.N, case.cfg.hkv, top_k), torch.int32)
    g_ro, ro = _guarded((tree.n_steps, q.shape[1], 128), q.dtype)
    tas.spec_qsa_attn_fwd(tree, q, k, v, to_device(idx["qi"]), to_device(idx["ki"]), G, top_k,
                          rope_base=case.cfg.rope_base, out=out, selected=sel, readout_out=ro)
    for name, gb in (("out", g_out), ("selected", g_sel), ("readout", g_ro)):
        _check(name, gb)
