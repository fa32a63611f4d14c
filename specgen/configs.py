"""Workload table for the branch-parallel scoring path.

Five named workloads (tiny, 8B-like GQA, long trunk, batched small trees,
stress) plus a constructor for small parity cases. Everything here is shape
and distribution metadata; the draws themselves live in ``specgen.gen``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    n_trees: int
    trunk: int                 # trunk length T of every tree
    branches: int              # anchors (branches) per tree
    width: int                 # branch width W (maximum when width_mode == "uniform")
    width_mode: str            # "fixed" or "uniform" (W_b ~ U{1..width})
    anchor_lo: int             # anchors are drawn from {anchor_lo .. T-1}
    anchor_replace: bool       # i.i.d. with replacement, else without
    hq: int
    hkv: int
    head_dim: int
    qkv_dtype: str             # "f32" or "bf16"
    rope_base: float
    vocab: int
    logit_dtype: str           # "f32" or "bf16"
    # logit recipe: ("iid", draft_std, teacher_std) -> independent draws
    #               ("noisy", draft_std, noise_std) -> teacher = draft + noise
    logits: Tuple[str, float, float]
    zipf_bias: Optional[float] = None   # exponent s of a -s*ln(v+1) bias on both
    seed: int = 0
    description: str = field(default="", compare=False)


CONFIGS = {
    "tiny": Config(
        name="tiny", n_trees=1, trunk=64, branches=4, width=4, width_mode="fixed",
        anchor_lo=8, anchor_replace=True, hq=4, hkv=2, head_dim=32, qkv_dtype="f32",
        rope_base=10000.0, vocab=512, logit_dtype="f32", logits=("iid", 2.0, 2.0),
        description="trunk 64, B=4 anchors U[8,63], W=4, 4q/2kv heads, D=32, fp32; V=512"),
    "gqa8b": Config(
        name="gqa8b", n_trees=1, trunk=4096, branches=256, width=16, width_mode="fixed",
        anchor_lo=8, anchor_replace=False, hq=32, hkv=8, head_dim=128, qkv_dtype="bf16",
        rope_base=10000.0, vocab=151936, logit_dtype="bf16", logits=("noisy", 3.0, 1.0),
        description="8B-like GQA: trunk 4096, B=256, W=16, 32q/8kv, D=128, bf16; "
                    "V=151936, teacher = draft + N(0,1)"),
    "long": Config(
        name="long", n_trees=1, trunk=16384, branches=512, width=16, width_mode="fixed",
        anchor_lo=8, anchor_replace=False, hq=32, hkv=8, head_dim=128, qkv_dtype="bf16",
        rope_base=10000.0, vocab=151936, logit_dtype="bf16", logits=("noisy", 3.0, 0.5),
        description="long trunk 16384, B=512, W=16, 32q/8kv, D=128, bf16; 8192 rows, "
                    "teacher = draft + N(0,0.5^2)"),
    "batched": Config(
        name="batched", n_trees=8, trunk=2048, branches=128, width=8, width_mode="fixed",
        anchor_lo=8, anchor_replace=False, hq=32, hkv=8, head_dim=128, qkv_dtype="bf16",
        rope_base=10000.0, vocab=151936, logit_dtype="bf16", logits=("iid", 3.0, 3.0),
        description="8 trees x (trunk 2048, B=128, W=8), 32q/8kv, D=128, bf16; "
                    "teacher independent N(0,3^2)"),
    "stress": Config(
        name="stress", n_trees=1, trunk=32768, branches=2048, width=16, width_mode="uniform",
        anchor_lo=8, anchor_replace=False, hq=64, hkv=8, head_dim=128, qkv_dtype="bf16",
        rope_base=10000.0, vocab=151936, logit_dtype="bf16", logits=("noisy", 3.0, 1.0),
        zipf_bias=1.1,
        description="trunk 32768, B=2048, W_b ~ U{1..16}, 64q/8kv, D=128, bf16; "
                    "Zipf(1.1) logit bias on both distributions"),
}

ORDER = ["tiny", "gqa8b", "long", "batched", "stress"]


def get_config(name: str) -> Config:
    return CONFIGS[name]


def small_config(name: str, **overrides) -> Config:
    """A reduced parity case: same recipe as ``name`` with sizes overridden."""
    return replace(CONFIGS[name], name=overrides.pop("tag", name + "_small"), **overrides)
