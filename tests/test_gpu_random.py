"""GPU: seeded random trees through the attention and E2E-TV paths, against the oracle.

Each case draws a forest (one to three trees; trunks of 1..200 tokens; 0..8 anchors per
tree, repeats allowed, anchored anywhere in the trunk; branch lengths 1..24 and now and
then the ABI maximum 64), a head layout (GQA groups 1, 3, 4, 8; head dims 64 and 128;
bf16 or float32), and a vocabulary (3 .. 30,000, bf16 or float32 logits), and compares
every output element with the float64 oracle at the tolerances of the other parity
tests."""
import numpy as np
import pytest

from _util import ATTN_ATOL, ATTN_ATOL_F32, Case, say
from specgen import small_config
from test_gpu_attn import _full_compare as attn_compare
from test_gpu_e2etv import _full_compare as e2etv_compare

pytestmark = pytest.mark.gpu

HEADS = [(8, 2, 128), (16, 2, 128), (4, 4, 64), (6, 2, 128), (8, 1, 64), (12, 4, 64), (16, 4, 128)]
VOCABS = [3, 100, 1000, 4104, 8191, 30000]


def _random_case(i):
    rng = np.random.default_rng(7000 + i)
    n_trees = int(rng.integers(1, 4))
    trunk = rng.integers(1, 201, size=n_trees).astype(np.int32)
    nb = rng.integers(0, 9, size=n_trees).astype(np.int32)
    anchors, widths = [], []
    for t in range(n_trees):
        anchors.append(rng.integers(0, trunk[t], size=nb[t]))
        w = rng.integers(1, 25, size=nb[t])
        w[rng.random(nb[t]) < 0.1] = 64
        widths.append(w)
    s = dict(trunk_len=trunk, n_branches=nb, anchors=np.concatenate(anchors).astype(np.int32),
             branch_len=np.concatenate(widths).astype(np.int32))
    hq, hkv, d = HEADS[i % len(HEADS)]
    qkv = "f32" if i % 5 == 4 else "bf16"
    vocab = VOCABS[i % len(VOCABS)]
    logit = "f32" if i % 4 == 3 else "bf16"
    cfg = small_config("gqa8b", hq=hq, hkv=hkv, head_dim=d, qkv_dtype=qkv, vocab=vocab, logit_dtype=logit,
                       seed=7000 + i)
    return Case(cfg, structure=s), (n_trees, hq, hkv, d, qkv, vocab, logit)


@pytest.mark.parametrize("i", range(12))
def test_random_forest(i):
    case, desc = _random_case(i)
    say("random forest %d: trees %d, heads %d/%d, D %d, %s, V %d, %s logits; N=%d R=%d"
        % ((i,) + desc + (case.N, case.R)))
    attn_compare(case, ATTN_ATOL_F32 if case.cfg.qkv_dtype == "f32" else ATTN_ATOL)
    if case.R > 0:
        z, y = case.logits()
        e2etv_compare(case, z, y)
