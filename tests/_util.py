"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np

from specgen import bf16_bits_to_f32, gen_logits, gen_qkv, gen_structure

ATTN_ATOL = 2e-2          # bf16 attention outputs, absolute
ATTN_ATOL_F32 = 1e-4      # float32 attention path, absolute
ALPHA_RTOL = 1e-5         # alpha, relative
LOSS_RTOL = 1e-5          # L, relative (absolute floor below)
LOSS_ATOL = 1e-7
GRAD_RTOL = 1e-4          # per row: max|g - g*| <= 1e-4 * max|g*|
TIE_MARGIN = 1e-5         # |ln q - ln p| below this: either one-sided derivative is valid


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns or float32 values -> float64 values (exact)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def to_device(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_device(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


class Case:
    """Structure plus lazily generated inputs of one workload."""

    def __init__(self, cfg, structure=None):
        self.cfg = cfg
        self.s = structure if structure is not None else gen_structure(cfg)
        from oracle import pack_ref
        self.lay = pack_ref(self.s["trunk_len"], self.s["n_branches"], self.s["anchors"],
                            self.s["branch_len"])
        self.N, self.R = self.lay["n_rows"], self.lay["n_steps"]
        self._qkv = None
        self._logits = None

    def qkv(self):
        if self._qkv is None:
            self._qkv = gen_qkv(self.cfg, self.N)
        return self._qkv

    def logits(self):
        if self._logits is None:
            self._logits = gen_logits(self.cfg, self.R)
        return self._logits

    def drop_logits(self):
        self._logits = None


def sample_rows(lay, k: int, seed: int = 0) -> np.ndarray:
    """Packed rows to check at full size: block edges, anchors, branch rows, random."""
    N = lay["n_rows"]
    rng = np.random.default_rng(seed)
    picks = {0, N - 1, 31, 32, 63, 64}
    for t in range(len(lay["tree_off"]) - 1):
        picks.add(int(lay["tree_off"][t]))
        picks.add(int(lay["tree_off"][t + 1]) - 1)
    br = np.flatnonzero(lay["row_branch"] >= 0)
    if br.size:
        picks.update(int(x) for x in br[:3])
        picks.update(int(x) for x in br[-3:])
        picks.update(int(x) for x in rng.choice(br, size=min(k // 2, br.size), replace=False))
    picks.update(int(x) for x in rng.choice(N, size=min(k // 2, N), replace=False))
    return np.array(sorted(p for p in picks if 0 <= p < N), dtype=np.int64)


S_ULPS = 2.0 ** -20        # absolute error allowed in the float32 S a gradient row is formed from


def check_grad_rows(g_gpu, g_ref, q, p, c=None, rtol=GRAD_RTOL):
    """Normwise per-row gradient check, skipping near-tie elements. Returns (worst, n_skipped).

    The gradient of a row is c q (1[q < p] - S). The kernels form S as a float32 sum of
    float32 exponentials, so S carries an absolute error of a few float32 ulps of 1, and
    the in-set coefficient c (1 - S) an absolute error of about |c| times that. When S
    lies within ~1e-4 of 1 (a draft whose mass sits almost entirely where the teacher is
    more confident: seen with three-token vocabularies, never on the workloads, where
    1 - S >= 0.54) the whole row is of that size. With the row coefficients `c` given,
    a row's scale is therefore at least S_ULPS / rtol * |c| * max_u q_u: the error
    allowed is at least S_ULPS |c| max q, eight float32 ulps of 1."""
    with np.errstate(divide="ignore", invalid="ignore"):
        lq, lp = np.log(q), np.log(p)
    tie = np.abs(lq - lp) <= TIE_MARGIN
    worst = 0.0
    for r in range(g_ref.shape[0]):
        scale = np.abs(g_ref[r]).max()
        if c is not None:
            scale = max(scale, S_ULPS / rtol * abs(float(c[r])) * float(np.max(q[r])))
        err = np.abs(np.where(tie[r], 0.0, g_gpu[r] - g_ref[r])).max()
        rel = err / scale if scale > 0 else err
        worst = max(worst, rel)
    return worst, int(tie.sum())
