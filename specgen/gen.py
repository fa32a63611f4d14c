"""Seeded synthetic draws.

Every array is drawn from NumPy's PCG64 seeded by
``SeedSequence(seed, spawn_key=(stream, chunk))``: the stream names the
tensor (0 structure, 1 Q, 2 K, 3 V, 4 draft logits, 5 teacher logits, 6-11
GDN inputs, 12-14 hidden states, output head and draft logits of the head
workloads) and the chunk is a fixed block of rows. Any chunk can therefore be regenerated alone
(the oracle uses this to rebuild sampled logit rows), and the bytes do not
depend on how many threads fill the chunks.

bfloat16 tensors are returned as their raw 16-bit patterns (``uint16``),
obtained from float32 draws by round-to-nearest-even.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Config

QKV_CHUNK_ROWS = 128
LOGIT_CHUNK_ROWS = 8

_S_STRUCT, _S_Q, _S_K, _S_V, _S_DRAFT, _S_TEACHER = range(6)
_S_GDN_Q, _S_GDN_K, _S_GDN_V, _S_GDN_TAPS, _S_GDN_GATES, _S_GDN_STATE = range(6, 12)
_S_HIDDEN, _S_HEAD, _S_HEAD_DRAFT = range(12, 15)
_S_QSA_QI, _S_QSA_KI = range(15, 17)
HEAD_CHUNK_ROWS = 1024


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream, chunk)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- structure

def gen_structure(cfg: Config):
    """Trunk lengths, branches per tree, local zero-based anchors and branch widths.

    Draw order: the anchors of every tree (tree by tree), then all branch widths.
    """
    g = _rng(cfg.seed, _S_STRUCT)
    trunk_len = np.full(cfg.n_trees, cfg.trunk, dtype=np.int32)
    n_branches = np.full(cfg.n_trees, cfg.branches, dtype=np.int32)
    anchors = []
    for _ in range(cfg.n_trees):
        lo, hi = cfg.anchor_lo, cfg.trunk            # anchors in {lo .. T-1}
        if cfg.anchor_replace:
            a = g.integers(lo, hi, size=cfg.branches)
        else:
            a = g.choice(np.arange(lo, hi), size=cfg.branches, replace=False)
        anchors.append(np.asarray(a, dtype=np.int32))
    anchors = np.concatenate(anchors) if anchors else np.zeros(0, np.int32)
    nb = cfg.n_trees * cfg.branches
    if cfg.width_mode == "fixed":
        widths = np.full(nb, cfg.width, dtype=np.int32)
    elif cfg.width_mode == "uniform":
        widths = g.integers(1, cfg.width + 1, size=nb).astype(np.int32)
    else:
        raise ValueError(cfg.width_mode)
    return dict(trunk_len=trunk_len, n_branches=n_branches,
                anchors=anchors.astype(np.int32), branch_len=widths)


# ----------------------------------------------------------------------------- Q / K / V

def _fill_normal(out_rows: np.ndarray, seed: int, stream: int, chunk: int, bf16: bool):
    x = _rng(seed, stream, chunk).standard_normal(out_rows.shape, dtype=np.float32)
    out_rows[...] = f32_to_bf16_bits(x) if bf16 else x


def gen_qkv(cfg: Config, n_rows: int):
    """Q [N,Hq,D], K [N,Hkv,D], V [N,Hkv,D], each element N(0,1).

    Returned as uint16 bfloat16 bit patterns or float32, per ``cfg.qkv_dtype``.
    """
    bf16 = cfg.qkv_dtype == "bf16"
    dt = np.uint16 if bf16 else np.float32
    q = np.empty((n_rows, cfg.hq, cfg.head_dim), dtype=dt)
    k = np.empty((n_rows, cfg.hkv, cfg.head_dim), dtype=dt)
    v = np.empty((n_rows, cfg.hkv, cfg.head_dim), dtype=dt)
    jobs = []
    for stream, arr in ((_S_Q, q), (_S_K, k), (_S_V, v)):
        for c, r0 in enumerate(range(0, n_rows, QKV_CHUNK_ROWS)):
            jobs.append((arr[r0:r0 + QKV_CHUNK_ROWS], stream, c))
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(lambda j: _fill_normal(j[0], cfg.seed, j[1], j[2], bf16), jobs))
    return q, k, v


# ----------------------------------------------------------------------------- logits

def _zipf_bias(cfg: Config) -> np.ndarray:
    v = np.arange(cfg.vocab, dtype=np.float64)
    return (-cfg.zipf_bias * np.log1p(v)).astype(np.float32)


def _logit_chunk(cfg: Config, chunk: int, nrows: int, bias):
    """Draft and teacher rows of one chunk as float32 values already rounded to the dtype."""
    bf16 = cfg.logit_dtype == "bf16"
    kind, s1, s2 = cfg.logits
    z = _rng(cfg.seed, _S_DRAFT, chunk).standard_normal((nrows, cfg.vocab), dtype=np.float32)
    z *= np.float32(s1)
    if bias is not None:
        z += bias
    if bf16:
        z = bf16_bits_to_f32(f32_to_bf16_bits(z))
    n2 = _rng(cfg.seed, _S_TEACHER, chunk).standard_normal((nrows, cfg.vocab), dtype=np.float32)
    n2 *= np.float32(s2)
    if kind == "iid":
        y = n2
    elif kind == "noisy":
        y = z + n2
    else:
        raise ValueError(kind)
    if bf16:
        y = bf16_bits_to_f32(f32_to_bf16_bits(y))
    return z, y


def gen_logits(cfg: Config, n_steps: int):
    """Draft and teacher logits [R, V], rows aligned with supervised steps.

    Returned as uint16 bfloat16 bit patterns or float32, per ``cfg.logit_dtype``.
    """
    bf16 = cfg.logit_dtype == "bf16"
    dt = np.uint16 if bf16 else np.float32
    draft = np.empty((n_steps, cfg.vocab), dtype=dt)
    teacher = np.empty((n_steps, cfg.vocab), dtype=dt)
    bias = _zipf_bias(cfg) if cfg.zipf_bias is not None else None

    def job(c):
        r0 = c * LOGIT_CHUNK_ROWS
        n = min(LOGIT_CHUNK_ROWS, n_steps - r0)
        z, y = _logit_chunk(cfg, c, n, bias)
        if bf16:
            draft[r0:r0 + n] = f32_to_bf16_bits(z)
            teacher[r0:r0 + n] = f32_to_bf16_bits(y)
        else:
            draft[r0:r0 + n] = z
            teacher[r0:r0 + n] = y

    nchunks = (n_steps + LOGIT_CHUNK_ROWS - 1) // LOGIT_CHUNK_ROWS
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(nchunks)))
    return draft, teacher


def gen_logit_rows(cfg: Config, n_steps: int, rows):
    """Regenerate only the given logit rows, as float32 values: (draft [k,V], teacher [k,V])."""
    rows = np.asarray(rows, dtype=np.int64)
    bias = _zipf_bias(cfg) if cfg.zipf_bias is not None else None
    out_z = np.empty((len(rows), cfg.vocab), np.float32)
    out_y = np.empty((len(rows), cfg.vocab), np.float32)
    cache = {}
    for i, r in enumerate(rows):
        c = int(r) // LOGIT_CHUNK_ROWS
        if c not in cache:
            r0 = c * LOGIT_CHUNK_ROWS
            cache[c] = _logit_chunk(cfg, c, min(LOGIT_CHUNK_ROWS, n_steps - r0), bias)
        z, y = cache[c]
        out_z[i] = z[int(r) - c * LOGIT_CHUNK_ROWS]
        out_y[i] = y[int(r) - c * LOGIT_CHUNK_ROWS]
    return out_z, out_y


# ----------------------------------------------------------------------------- GDN replay inputs

def gen_gdn(seed: int, n_rows: int, heads: int, head_dim: int, conv_width: int):
    """Inputs of the indexed GDN replay on a packed tree of n_rows rows.

    Returns a dict:
      xq, xk, xv  [N, H, D] uint16 bfloat16 bits, N(0,1): projections before the
                  short convolution, for every packed row;
      taps        [3, H, D, K] float32, N(0, 0.5^2): convolution taps of q, k, v
                  (tap j on the j-th ancestor);
      alpha       [N, H] float32, U(0.9, 1.0): per-token decay;
      beta        [N, H] float32, U(0.05, 0.95): per-token write strength.
    """
    out = {}
    for name, stream in (("xq", _S_GDN_Q), ("xk", _S_GDN_K), ("xv", _S_GDN_V)):
        arr = np.empty((n_rows, heads, head_dim), dtype=np.uint16)
        jobs = [(arr[r0:r0 + QKV_CHUNK_ROWS], c) for c, r0 in enumerate(range(0, n_rows, QKV_CHUNK_ROWS))]
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(lambda j, st=stream: _fill_normal(j[0], seed, st, j[1], True), jobs))
        out[name] = arr
    g = _rng(seed, _S_GDN_TAPS)
    out["taps"] = (0.5 * g.standard_normal((3, heads, head_dim, conv_width))).astype(np.float32)
    g = _rng(seed, _S_GDN_GATES)
    out["alpha"] = g.uniform(0.9, 1.0, size=(n_rows, heads)).astype(np.float32)
    out["beta"] = g.uniform(0.05, 0.95, size=(n_rows, heads)).astype(np.float32)
    return out


def gen_gdn_states(seed: int, n_states: int, heads: int, head_dim: int, std: float = 0.2):
    """n_states synthetic float32 GDN states [n_states, H, D, D], N(0, std^2), as
    stand-in checkpoints where a trunk pass is not run."""
    st = np.empty((n_states, heads, head_dim, head_dim), dtype=np.float32)

    def fill(i):
        st[i] = np.float32(std) * _rng(seed, _S_GDN_STATE, i).standard_normal(
            (heads, head_dim, head_dim), dtype=np.float32)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(n_states)))
    return st


def _fill_scaled_bf16(out_rows: np.ndarray, seed: int, stream: int, chunk: int, std: float):
    x = _rng(seed, stream, chunk).standard_normal(out_rows.shape, dtype=np.float32)
    out_rows[...] = f32_to_bf16_bits(np.float32(std) * x)


def _chunked_bf16(shape, chunk_rows: int, seed: int, stream: int, std: float) -> np.ndarray:
    arr = np.empty(shape, dtype=np.uint16)
    jobs = [(arr[r0:r0 + chunk_rows], c) for c, r0 in enumerate(range(0, shape[0], chunk_rows))]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(lambda j: _fill_scaled_bf16(j[0], seed, stream, j[1], std), jobs))
    return arr


def gen_head(seed: int, n_rows: int, d_model: int, vocab: int, n_steps: int, logit_std: float = 3.0):
    """Inputs of E2E-TV scored from hidden states through an output head.

    Returns a dict of uint16 bfloat16 bit patterns:
      hidden  [N, d_model] N(0,1): final hidden states of every packed row;
      head    [V, d_model] N(0, (logit_std / sqrt(d_model))^2): the output head,
              so that a teacher logit has standard deviation about logit_std;
      draft   [R, V] N(0, logit_std^2): draft logits, one row per supervised step.
    """
    return {
        "hidden": _chunked_bf16((n_rows, d_model), HEAD_CHUNK_ROWS, seed, _S_HIDDEN, 1.0),
        "head": _chunked_bf16((vocab, d_model), HEAD_CHUNK_ROWS, seed, _S_HEAD,
                              logit_std / np.sqrt(d_model)),
        "draft": _chunked_bf16((n_steps, vocab), LOGIT_CHUNK_ROWS, seed, _S_HEAD_DRAFT, logit_std),
    }


def gen_head_draft_rows(seed: int, n_steps: int, vocab: int, rows, logit_std: float = 3.0):
    """Regenerate only the given rows of gen_head's draft logits (bf16 bit patterns [k, V])."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), vocab), dtype=np.uint16)
    for c in np.unique(rows // LOGIT_CHUNK_ROWS):
        n = min(LOGIT_CHUNK_ROWS, n_steps - c * LOGIT_CHUNK_ROWS)
        blk = np.empty((n, vocab), dtype=np.uint16)
        _fill_scaled_bf16(blk, seed, _S_HEAD_DRAFT, int(c), logit_std)
        sel = rows // LOGIT_CHUNK_ROWS == c
        out[sel] = blk[rows[sel] - c * LOGIT_CHUNK_ROWS]
    return out


def _fill_grid_bf16(out_rows: np.ndarray, seed: int, stream: int, chunk: int, levels: int):
    x = _rng(seed, stream, chunk).integers(-levels, levels + 1, size=out_rows.shape)
    out_rows[...] = f32_to_bf16_bits((x / np.float32(levels)).astype(np.float32))


def gen_qsa_index(seed: int, n_rows: int, n_heads_kv: int, index_dim: int, grid: int = 0):
    """Indexer queries and keys of sparse attention: [N, Hkv, DI] each, bf16 bit patterns.

    grid = 0: N(0,1) draws. grid = m > 0: values k/m for integers k in [-m, m]
    (exactly representable in bf16), so that with a power-of-two group size every
    group mean and every score is exact in float32 as well as in float64.
    """
    out = {}
    for name, stream in (("qi", _S_QSA_QI), ("ki", _S_QSA_KI)):
        arr = np.empty((n_rows, n_heads_kv, index_dim), dtype=np.uint16)
        jobs = [(arr[r0:r0 + QKV_CHUNK_ROWS], c) for c, r0 in enumerate(range(0, n_rows, QKV_CHUNK_ROWS))]
        if grid:
            fill = lambda j: _fill_grid_bf16(j[0], seed, stream, j[1], grid)
        else:
            fill = lambda j: _fill_scaled_bf16(j[0], seed, stream, j[1], 1.0)
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, jobs))
        out[name] = arr
    return out
