#!/usr/bin/env python3
"""Benchmark of the branch-parallel scoring step on one MI355X.

One step is the whole hot path over one packed proposal tree: pack (host plan,
copy, expand), tree attention with RoPE and readout, then the E2E-TV forward
and backward over the supervised rows. Inputs are seeded synthetic tensors,
already resident in device memory when the timed region starts. The headline
is supervised rows per second; per-kernel durations come from HIP events
recorded by the library on the stream it launches on, inside the timed steps.

    python bench.py [--steps K] [--warmup W] [--config stress] [--no-cpu-baseline]
    python bench.py --gdn [--config gqa8b]   # GDN scoring: trunk pass + indexed replay
    python bench.py --head [--config gqa8b]  # E2E-TV through the output head
    python bench.py --qsa [--config gqa8b]   # sparse attention with branch-consistent indexer groups

The default workload is the stress tree (trunk 32768, 2048 branches of 1..16
steps, 64 query / 8 KV heads, vocabulary 151936): the largest of the five
workloads, all of which fit one GPU.

Prints one JSON line. Only one GPU is supported (--gpus must be 1).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def causal_pairs(s) -> int:
    """Visible (query, key) pairs: trunk triangles plus each branch row's prefix."""
    import numpy as np
    P = int(sum(int(t) * (int(t) + 1) // 2 for t in s["trunk_len"]))
    a = s["anchors"].astype(np.int64)
    w = s["branch_len"].astype(np.int64)
    # sum_{i=1}^{W-1} (a + 1 + i) = (W-1)(a+1) + (W-1)W/2
    P += int(np.sum((w - 1) * (a + 1) + (w - 1) * w // 2))
    return P


def source_hash(*names) -> str:
    """Hash of the named library sources and the header they all share."""
    h = hashlib.sha256()
    for n in ("common.h",) + names:
        with open(os.path.join(ROOT, "tree_attention_spec_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, src_hash: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on this workload and the kernel's source has not changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


# Library timing marks -> the kernels each covers (matched by substring of the
# kernel name rocprofv3 records) and the source files whose hash keys its
# measured traffic (the attention kernel reads tiles laid out by rope.hip).
MARK_KERNELS = {
    "tree_attn": (["tree_attn_tiled_kernel", "tree_attn_bf16_kernel", "tree_attn_f32_kernel"],
                  ("attn.hip", "rope.hip")),
    "rope_k": (["rope_k_kernel"], ("rope.hip",)),
    "kv_tiles": (["kv_tile_kernel"], ("rope.hip",)),
    "readout": (["readout_kernel"], ("attn.hip",)),
    "e2etv_clear": (["e2etv_fuse_clear"], ("e2etv.hip",)),
    "e2etv_fused": (["e2etv_fused_team_kernel"], ("e2etv.hip",)),
    "e2etv_loss": (["e2etv_loss_kernel"], ("e2etv.hip",)),
    "e2etv_stats": (["e2etv_team_clear", "e2etv_stats_team_kernel", "e2etv_stats_kernel"], ("e2etv.hip",)),
    "e2etv_scan": (["e2etv_scan_kernel"], ("e2etv.hip",)),
    "e2etv_grad": (["e2etv_grad_kernel"], ("e2etv.hip",)),
    "e2etv_head_lse": (["e2etv_head_lse_kernel"], ("e2etv_head.hip",)),
    "e2etv_head_merge": (["e2etv_head_merge_kernel"], ("e2etv_head.hip",)),
    "e2etv_head_tv": (["e2etv_head_tv_kernel"], ("e2etv_head.hip",)),
    "e2etv_head_sum": (["e2etv_head_sum_kernel"], ("e2etv_head.hip",)),
    "gdn_trunk": (["gdn_trunk_kernel"], ("gdn.hip", "gdn_util.h")),
    "gdn_chunk_prep": (["gdn_chunk_prep_kernel"], ("gdn_chunk.hip", "gdn_util.h")),
    "gdn_chunk_scan": (["gdn_chunk_scan_kernel"], ("gdn_chunk.hip", "gdn_util.h")),
    "gdn_chunk_out": (["gdn_chunk_out_kernel"], ("gdn_chunk.hip", "gdn_util.h")),
    "gdn_replay": (["gdn_replay_kernel"], ("gdn.hip", "gdn_util.h")),
    "gdn_replay_chunk": (["gdn_replay_chunk_kernel"], ("gdn_chunk.hip", "gdn_util.h")),
    "qsa_keys": (["qsa_keys_kernel"], ("qsa.hip",)),
    "qsa_select": (["qsa_select_kernel"], ("qsa.hip",)),
    "qsa_attn": (["qsa_attn_kernel"], ("qsa.hip", "rope.hip")),
}


def write_traffic(fetch_db, write_db, copy_fetch_db, copy_write_db, workload):
    """profiles/traffic.json from FETCH_SIZE / WRITE_SIZE runs, scaled by a 1 GiB copy.

    Entries for kernels the runs did not launch are kept as they were."""
    pm = summarize_pmc([fetch_db, write_db])
    cp = summarize_pmc([copy_fetch_db, copy_write_db])
    copy = next(v for k, v in cp.items() if "copyBuffer" in k)
    n = 1 << 30
    fs = n / (copy["FETCH_SIZE"]["mean"] * 1024.0)
    ws = n / (copy["WRITE_SIZE"]["mean"] * 1024.0)
    try:
        with open(TRAFFIC_FILE) as f:
            out = json.load(f)
    except (OSError, ValueError):
        out = {}
    out["_calibration"] = {"copy_bytes": n, "fetch_kib": copy["FETCH_SIZE"]["mean"],
                            "write_kib": copy["WRITE_SIZE"]["mean"], "fetch_scale": fs, "write_scale": ws,
                            "note": "1 GiB device copy (bench.py --copy-calibration)"}
    for mark, (subs, src) in MARK_KERNELS.items():
        ks = [v for k, v in pm.items() if any(sub in k for sub in subs)]
        if not ks:
            continue
        fk = sum(v.get("FETCH_SIZE", {}).get("mean", 0.0) for v in ks)
        wk = sum(v.get("WRITE_SIZE", {}).get("mean", 0.0) for v in ks)
        out[mark] = {"source_hash": source_hash(*src), "workload": workload,
                     "fetch_bytes": fk * 1024 * fs, "write_bytes": wk * 1024 * ws,
                     "bytes_per_launch": fk * 1024 * fs + wk * 1024 * ws,
                     "fetch_kib_raw": fk, "write_kib_raw": wk}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def summarize_pmc(paths):
    """Per-kernel mean of every counter in rocprofv3 --pmc databases (no GPU needed)."""
    import collections
    import sqlite3
    out = {}
    for path in paths:
        cur = sqlite3.connect(path).cursor()
        rows = cur.execute("select k.name, p.counter_name, p.counter_value from pmc_events p "
                           "join kernels k on p.dispatch_id = k.dispatch_id").fetchall()
        agg = collections.defaultdict(list)
        for name, counter, value in rows:
            agg[(name, counter)].append(value)
        for (name, counter), vals in sorted(agg.items()):
            out.setdefault(name, {})[counter] = {"dispatches": len(vals), "mean": sum(vals) / len(vals)}
    return out


def ablation(cfg, s, tree, qt, kt, vt, out, steps, warmup):
    """Shared-prefix scoring against uncached independent scoring, same kernel.

    The independent layout packs every branch as a tree of its own: the trunk
    through the branch's anchor, then the branch (the unpacked causal sequence of
    the branch). Q, K and V rows are gathered from the shared layout's rows, so
    both layouts score the same tokens at the same positions; the branch and
    anchor rows of both must agree up to summation order.
    """
    import numpy as np
    import torch
    import tree_attention_spec_amd as tas
    dev = qt.device
    lay = {k_: v_.cpu().numpy() for k_, v_ in tree.arrays().items()}
    a = s["anchors"].astype(np.int64)
    w = s["branch_len"].astype(np.int64)
    t_of_b = np.repeat(np.arange(len(s["trunk_len"])), s["n_branches"])
    trunk_rows = lay["tree_off"][t_of_b].astype(np.int64)
    idx = np.concatenate([np.concatenate([trunk_rows[b] + np.arange(a[b] + 1), lay["branch_off"][b] + np.arange(w[b] - 1)])
                          for b in range(len(a))])
    idx_t = torch.from_numpy(idx).to(dev)
    qi, ki, vi = qt.index_select(0, idx_t), kt.index_select(0, idx_t), vt.index_select(0, idx_t)
    tree_i = tas.spec_tree_pack((a + 1).astype(np.int32), np.ones(len(a), np.int32), a.astype(np.int32),
                                w.astype(np.int32), device=dev)
    out_i = torch.empty_like(qi)
    work_i = torch.empty(tas.attn_work_bytes(tree_i, cfg.hq, cfg.hkv, cfg.head_dim, qi.dtype), dtype=torch.uint8,
                         device=dev)

    def timed(tr, q_, k_, v_, o_, wk):
        for _ in range(warmup):
            tas.spec_tree_attn_fwd(tr, q_, k_, v_, rope_base=cfg.rope_base, out=o_, work=wk)
        per = {}
        for _ in range(steps):
            tm = tas.KernelTimer(capacity=16)
            with tm:
                tas.spec_tree_attn_fwd(tr, q_, k_, v_, rope_base=cfg.rope_base, out=o_, work=wk)
            for name, ms in tm.durations():
                per.setdefault(name, []).append(ms)
        return {n_: sum(x) / len(x) for n_, x in per.items()}

    work_s = torch.empty(tas.attn_work_bytes(tree, cfg.hq, cfg.hkv, cfg.head_dim, qt.dtype), dtype=torch.uint8,
                         device=dev)
    t_shared = timed(tree, qt, kt, vt, out, work_s)
    t_ind = timed(tree_i, qi, ki, vi, out_i, work_i)
    # branch rows and anchor rows of both layouts
    toff_i = tree_i.arrays()["tree_off"].cpu().numpy().astype(np.int64)
    rows_s, rows_i = [], []
    for b in range(len(a)):
        rows_s.append(np.concatenate([[trunk_rows[b] + a[b]], lay["branch_off"][b] + np.arange(w[b] - 1)]))
        rows_i.append(toff_i[b] + a[b] + np.arange(w[b]))
    rs = torch.from_numpy(np.concatenate(rows_s)).to(dev)
    ri = torch.from_numpy(np.concatenate(rows_i)).to(dev)
    diff = (out.index_select(0, rs).float() - out_i.index_select(0, ri).float()).abs().max().item()
    p_shared = causal_pairs(s)
    p_ind = int(np.sum((a + 1) * (a + 2) // 2 + (w - 1) * (a + 1) + (w - 1) * w // 2))
    return {
        "what": "tree attention (RoPE + attention kernels) on the shared-prefix packed tree vs every branch "
                "scored as its own causal sequence (trunk through its anchor + its branch), same kernels",
        "shared": {"rows": int(tree.n_rows), "causal_pairs": p_shared, "kernel_ms": t_shared},
        "independent": {"rows": int(tree_i.n_rows), "causal_pairs": p_ind, "kernel_ms": t_ind},
        "pair_ratio": p_ind / p_shared,
        "attention_time_ratio": t_ind["tree_attn"] / t_shared["tree_attn"],
        "max_abs_diff_branch_and_anchor_rows": diff,
    }


def cpu_baseline(cfg, s, q, k, v, z_rows_fn, N, R, n_attn=None, n_e2e=6):
    """Time the oracle on a bounded random sample and scale it to the full step.

    The sample is spread over one thread per host CPU (at most 16): NumPy releases
    the interpreter lock inside its array operations, so each thread runs the
    oracle on its own share of rows. Every thread gets n_attn attention rows and
    n_e2e logit rows, so the wall time stays near that of one thread on the
    smaller sample while the sample grows with the thread count.
    """
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import e2etv_coef_ref, e2etv_grad_ref, e2etv_row_stats_ref, pack_ref, rope_ref, tree_attn_ref
    from specgen import bf16_bits_to_f32

    def widen(a):
        return bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    if n_attn is None:
        # a row's oracle cost grows with the keys it sees: fewer rows on long trunks keep
        # the sample near 10-30 s of host time
        n_attn = max(4, min(24, int(24 * 4096 / max(int(max(s["trunk_len"])), 1))))
    rng = np.random.default_rng(123)
    t0 = time.perf_counter()
    lay = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    t_pack = time.perf_counter() - t0
    qd, kd, vd = widen(q), widen(k), widen(v)
    with ThreadPoolExecutor(workers) as ex:
        # the K rotation every attention call repeats, timed on its own
        t0 = time.perf_counter()
        rope_ref(kd, lay["row_pos"][:, None], cfg.rope_base)
        t_fixed = time.perf_counter() - t0
        rows = rng.choice(N, size=min(n_attn * workers, N), replace=False)
        t0 = time.perf_counter()
        list(ex.map(lambda part: tree_attn_ref(lay, qd, kd, vd, cfg.rope_base, rows=part),
                    np.array_split(rows, workers)))
        t_call = time.perf_counter() - t0
        t_attn = t_fixed + (N / len(rows)) * max(t_call - t_fixed, 0.0)
        srows = np.sort(rng.choice(R, size=min(n_e2e * workers, R), replace=False))
        zs, ys = z_rows_fn(srows)

        def e2e(part):
            alpha, S, _, _, qq, pp = e2etv_row_stats_ref(zs[part].astype(np.float64), ys[part].astype(np.float64))
            c = e2etv_coef_ref(alpha, [0, len(part)])
            e2etv_grad_ref(qq, pp, S, c)

        t0 = time.perf_counter()
        list(ex.map(e2e, np.array_split(np.arange(len(srows)), workers)))
        t_e2e = (R / len(srows)) * (time.perf_counter() - t0)
    total = t_pack + t_attn + t_e2e
    return {
        "value": R / total, "unit": "supervised rows/s", "cores": workers, "kind": "oracle",
        "sample": "%d random packed rows of tree attention (plus the full K rotation) and %d random "
                  "logit rows of E2E-TV stats+gradient, float64 NumPy, spread over %d threads; scaled "
                  "to the full step (N=%d rows, R=%d steps)" % (len(rows), len(srows), workers, N, R),
        "seconds_full_step_estimate": total,
        "host_cpus": len(os.sched_getaffinity(0)),
    }


GDN_CONV_WIDTH, GDN_CHUNK = 4, 64


def gdn_work(s, C):
    """Replayed trunk tokens and branch tokens over all branches (one head)."""
    import numpy as np
    a = np.asarray(s["anchors"], np.int64)
    w = np.asarray(s["branch_len"], np.int64)
    replay = a - ((a + 1) // C) * C + 1
    return int(replay.sum()), int(np.maximum(w - 1, 0).sum())


def gdn_flops(s, H, D, C):
    """Algorithmic flops of each GDN kernel (an FMA counts two).

    Token-at-a-time (trunk pass with C > 64, and the replay): per token and head
    u = S k (D^2 FMA) and S <- alpha S + w k^T (D^2 mul + D^2 FMA), plus o = S q
    (D^2 FMA) for a token whose output is read. Chunked trunk pass, per chunk of
    L tokens and head: prep forms A (L(L-1)/2 dots of length D) and P (L(L+1)/2
    dots), solves for the 2D columns of [U | W] (L(L-1)/2 FMAs each) and forms
    P [U | W] (L(L+1)/2 FMAs per column); scan (full chunks only) forms
    U - W S^T and delta^T Kd (L D^2 FMAs each); out forms Q' S^T (L D^2 FMAs)."""
    import numpy as np
    T = np.asarray(s["trunk_len"], np.int64)
    n_replay, n_branch = gdn_work(s, C)
    f = {"gdn_replay": float(H) * D * D * (5 * n_replay + 7 * n_branch),
         "gdn_trunk": float(H) * D * D * 7 * int(T.sum())}
    Ls = np.concatenate([np.minimum(C, t - np.arange(0, t, C)) for t in T]).astype(np.float64)
    full = Ls[Ls == C]
    tri = Ls * (Ls - 1) / 2 + Ls * (Ls + 1) / 2            # entries of A and P
    f["gdn_chunk_prep"] = float(H) * float(np.sum(2 * D * tri + 2 * 2 * D * tri))
    f["gdn_chunk_scan"] = float(H) * float(np.sum(2 * 2 * full * D * D))
    f["gdn_chunk_out"] = float(H) * float(np.sum(2 * Ls * D * D))
    # replay from the cache, per branch (m = W - 1 tokens, j replayed trunk tokens) and head:
    # the branch chunk's A, P, solve and P X as in prep, then Q' S_c^T (m D^2 FMAs),
    # Q' K'^T (m j D) and Y Delta (m j D)
    a = np.asarray(s["anchors"], np.int64)
    m = np.maximum(np.asarray(s["branch_len"], np.int64) - 1, 0).astype(np.float64)
    j = (a + 1 - ((a + 1) // C) * C).astype(np.float64)
    tri_b = m * (m - 1) / 2 + m * (m + 1) / 2
    f["gdn_replay_chunk"] = float(H) * float(np.sum((m > 0) * (6 * D * tri_b + 2 * m * D * D
                                                                + 4 * m * j * D)))
    return f


def gdn_bench(args, cfg, s, dev):
    """GDN scoring of the workload's tree: the shared trunk pass (trunk outputs and
    checkpoints every 64 tokens), then the indexed replay of every branch from those
    checkpoints; cfg.hq heads of cfg.head_dim and a width-4 convolution."""
    import numpy as np
    import torch
    import tree_attention_spec_amd as tas
    from specgen import gen_gdn

    H, D, K, C = cfg.hq, cfg.head_dim, GDN_CONV_WIDTH, GDN_CHUNK
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    N = tree.n_rows
    log("GDN scoring: N=%d rows, %d branches, H=%d, D=%d, K=%d, C=%d; generating inputs"
        % (N, tree.n_branches, H, D, K, C))
    inp = gen_gdn(cfg.seed, N, H, D, K)
    slots = tas.gdn_checkpoint_slots(tree, C)
    t = {}
    for name in ("xq", "xk", "xv"):
        t[name] = torch.from_numpy(inp[name].view(np.int16)).to(dev).view(torch.bfloat16)
    for name in ("taps", "alpha", "beta"):
        t[name] = torch.from_numpy(inp[name]).to(dev)
    x = [t[n] for n in ("xq", "xk", "xv", "taps", "alpha", "beta")]
    ckpt = torch.zeros((tree.n_trees, slots, H, D, D), dtype=torch.float32, device=dev)
    out = torch.zeros((N, H, D), dtype=torch.float32, device=dev)
    work = torch.empty(tas.gdn_trunk_work_bytes(tree, H, D, K, C), dtype=torch.uint8, device=dev)

    def call():
        tas.spec_gdn_trunk_fwd(tree, *x, chunk=C, ckpt=ckpt, out=out, work=work)
        tas.spec_gdn_replay_fwd(tree, *x, ckpt=ckpt, chunk=C, out=out,
                                trunk_work=None if args.gdn_token_replay else work)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    timers = [tas.KernelTimer(capacity=8) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        with timers[i]:
            call()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {}
    for tm in timers:
        for n, d in tm.durations():
            per.setdefault(n, []).append(d)
    kms = {n: sum(v) / len(v) for n, v in per.items()}
    n_replay, n_branch = gdn_work(s, C)
    n_trunk = int(np.sum(s["trunk_len"]))
    flop = gdn_flops(s, H, D, C)
    tf = {k: flop[k] / (kms[k] * 1e-3) / 1e12 for k in kms}
    for k in kms:
        log("%s %.4f ms (%.1f TFLOP/s)" % (k, kms[k], tf[k]))
    rk = "gdn_replay" if args.gdn_token_replay else "gdn_replay_chunk"
    log("trunk pass %.4f ms, replay %.4f ms" % (sum(v for k, v in kms.items() if k != rk), kms[rk]))
    log("per head: %d trunk tokens, %d replayed + %d branch tokens" % (n_trunk, n_replay, n_branch))
    dom = max(kms, key=kms.get)
    return {
        "metric": "GDN tree scoring rows/s (trunk pass + indexed replay, all heads)",
        "value": N / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded inputs)",
        "config": {"workload": cfg.name + " tree, GDN scoring", "n_rows": N, "branches": tree.n_branches,
                   "heads": H, "head_dim": D, "conv_width": K, "chunk": C, "trunk_tokens": n_trunk,
                   "replayed_tokens": n_replay, "branch_tokens": n_branch, "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": "alu", "achieved": tf[dom],
                     "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s", "frac": tf[dom] / PEAK_F32_TFLOPS,
                     "algorithmic_flop_per_launch": flop[dom],
                     "traffic": measured_traffic(dom, source_hash(*MARK_KERNELS[dom][1]), args.config)},
        "kernels": {k: {"ms": kms[k], "tflops": tf[k], "frac": tf[k] / PEAK_F32_TFLOPS,
                        "traffic": measured_traffic(k, source_hash(*MARK_KERNELS[k][1]), args.config)}
                    for k in kms},
        **({} if args.no_cpu_baseline else
           {"cpu_baseline": gdn_cpu_baseline(s, inp, C, N)}),
    }


def head_bench(args, cfg, s, dev):
    """E2E-TV scored from hidden states through an output head (readout, head product and
    E2E-TV fused; teacher logits never stored): the workload's supervised steps, hidden size
    cfg.hq * cfg.head_dim, vocabulary cfg.vocab, bf16 draft logits, gradient written."""
    import numpy as np
    import torch
    import tree_attention_spec_amd as tas
    from specgen import gen_head

    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    N, R, V, d = tree.n_rows, tree.n_steps, cfg.vocab, cfg.hq * cfg.head_dim
    log("E2E-TV through the head: R=%d steps, N=%d rows, d_model=%d, V=%d; generating inputs"
        % (R, N, d, V))
    inp = gen_head(cfg.seed, N, d, V, R)
    x = {k: torch.from_numpy(inp[k].view(np.int16)).to(dev).view(torch.bfloat16)
         for k in ("draft", "hidden", "head")}
    alpha = torch.empty(R, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    grad = torch.empty((R, V), dtype=torch.float32, device=dev)
    work = torch.empty(tas.e2etv_head_work_bytes(tree, V, d), dtype=torch.uint8, device=dev)

    def call():
        tas.spec_e2etv_head_fwd_bwd(tree, x["draft"], x["hidden"], x["head"], alpha_out=alpha,
                                    loss_out=loss, grad_out=grad, work=work)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    timers = [tas.KernelTimer(capacity=12) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        with timers[i]:
            call()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {}
    for tm in timers:
        for n, dd in tm.durations():
            per.setdefault(n, []).append(dd)
    kms = {n: sum(v) / len(v) for n, v in per.items()}
    for k in kms:
        log("%s %.4f ms" % (k, kms[k]))
    gemm = 2.0 * R * d * V           # one pass of the head product
    dom = max(("e2etv_head_lse", "e2etv_head_tv"), key=kms.get)
    tf = gemm / (kms[dom] * 1e-3) / 1e12
    kern = {k: {"ms": kms[k], "traffic": measured_traffic(k, source_hash(*MARK_KERNELS[k][1]), args.config)}
            for k in kms if k in MARK_KERNELS}
    for k in ("e2etv_head_lse", "e2etv_head_tv"):
        kern[k]["tflops"] = gemm / (kms[k] * 1e-3) / 1e12
        kern[k]["frac"] = kern[k]["tflops"] / PEAK_BF16_TFLOPS
    return {
        "metric": "E2E-TV rows/s from hidden states and output head (fwd + grad)",
        "value": R / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded inputs)",
        "config": {"workload": cfg.name + " tree, E2E-TV through the output head", "steps": R,
                   "n_rows": N, "d_model": d, "vocab": V, "draft_dtype": "bf16",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                     "algorithmic_flop_per_launch": gemm,
                     "traffic": measured_traffic(dom, source_hash(*MARK_KERNELS[dom][1]), args.config)},
        "kernels": kern,
        **({} if args.no_cpu_baseline else {"cpu_baseline": head_cpu_baseline(s, inp, R)}),
    }


QSA_GROUP, QSA_TOP_K, QSA_INDEX_DIM = 64, 16, 64


def qsa_keys_read(s, G, top_k):
    """Keys every packed row attends to under sparse attention: the picked groups' G keys
    each (min(n_c, top_k) groups) plus the causal tail, summed over rows."""
    import numpy as np
    tot = 0
    for t_len in s["trunk_len"]:
        tot += _qsa_keys_at(np.arange(int(t_len), dtype=np.int64), G, top_k)
    a = np.asarray(s["anchors"], np.int64)
    w = np.asarray(s["branch_len"], np.int64)
    for ab, wb in zip(a, w):
        pos = ab + np.arange(1, wb, dtype=np.int64)
        tot += _qsa_keys_at(pos, G, top_k)
    return int(tot)


def _qsa_keys_at(pos, G, top_k):
    import numpy as np
    n_c = (pos + 1) // G
    return int(np.sum(np.minimum(n_c, top_k) * G + (pos + 1 - n_c * G)))


def qsa_bench(args, cfg, s, dev):
    """Sparse attention with branch-consistent indexer groups over the workload's tree:
    group keys, top-k picks and attention over the picked groups plus the causal tail
    (G = 64, top_k = 16, index dim 64, N(0,1) indexer inputs), with the readout."""
    import numpy as np
    import torch
    import tree_attention_spec_amd as tas
    from specgen import gen_qkv, gen_qsa_index

    G, K, DI = QSA_GROUP, QSA_TOP_K, QSA_INDEX_DIM
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    N = tree.n_rows
    log("sparse attention: N=%d rows, %d/%d heads, G=%d, top_k=%d, index dim %d; generating inputs"
        % (N, cfg.hq, cfg.hkv, G, K, DI))
    q, k, v = gen_qkv(cfg, N)
    idx = gen_qsa_index(cfg.seed, N, cfg.hkv, DI)
    dvt = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    qt, kt, vt, qit, kit = dvt(q), dvt(k), dvt(v), dvt(idx["qi"]), dvt(idx["ki"])
    out = torch.empty_like(qt)
    sel = torch.empty((N, cfg.hkv, K), dtype=torch.int32, device=dev)
    ro = torch.empty((tree.n_steps, cfg.hq, cfg.head_dim), dtype=qt.dtype, device=dev)
    work = torch.empty(tas.qsa_work_bytes(tree, cfg.hq, cfg.hkv, cfg.head_dim, DI, G, K), dtype=torch.uint8,
                       device=dev)

    def call():
        tas.spec_qsa_attn_fwd(tree, qt, kt, vt, qit, kit, G, K, rope_base=cfg.rope_base, out=out, selected=sel,
                              readout_out=ro, work=work)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    timers = [tas.KernelTimer(capacity=12) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        with timers[i]:
            call()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {}
    for tm in timers:
        for n, d in tm.durations():
            per.setdefault(n, []).append(d)
    kms = {n: sum(x) / len(x) for n, x in per.items()}
    for kname in kms:
        log("%s %.4f ms" % (kname, kms[kname]))
    keys = qsa_keys_read(s, G, K)
    flop = 4.0 * cfg.head_dim * cfg.hq * keys
    gathered = float(keys) * cfg.hkv * cfg.head_dim * 2 * 2          # K and V bytes the rows read
    t_attn = kms.get("qsa_attn", float("nan"))
    tf = flop / (t_attn * 1e-3) / 1e12
    res = {
        "metric": "sparse-attention rows/s (group keys + top-k picks + attention over picked groups and tail)",
        "value": N / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded inputs)",
        "config": {"workload": cfg.name + " tree, sparse attention with branch-consistent indexer groups",
                   "n_rows": N, "heads_q": cfg.hq, "heads_kv": cfg.hkv, "head_dim": cfg.head_dim,
                   "group_size": G, "top_k": K, "index_dim": DI, "attended_keys": keys,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "qsa_attn", "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS, "algorithmic_flop_per_launch": flop,
                     "gathered_kv_bytes_per_launch": gathered,
                     "gathered_GBs": gathered / (t_attn * 1e-3) / 1e9,
                     "traffic": measured_traffic("qsa_attn", source_hash(*MARK_KERNELS["qsa_attn"][1]),
                                                 args.config)},
        "kernel_ms": kms,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = qsa_cpu_baseline(cfg, s, q, k, v, idx, G, K, N)
    return res


def qsa_cpu_baseline(cfg, s, q, k, v, idx, G, K, N, per_thread=2):
    """The sparse-attention oracle on a bounded sample: per_thread random packed rows per
    host thread (history walk, group keys, picks, attention), scaled to all rows."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import pack_ref
    from oracle.qsa_ref import qsa_attn_ref
    from specgen import bf16_bits_to_f32

    log("timing the sparse-attention oracle on a bounded sample")
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    lay = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    wid = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    qd, kd, vd, qid, kid = wid(q), wid(k), wid(v), wid(idx["qi"]), wid(idx["ki"])
    rows = np.random.default_rng(321).choice(N, size=min(N, per_thread * workers), replace=False)
    with ThreadPoolExecutor(workers) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda part: qsa_attn_ref(lay, qd, kd, vd, qid, kid, G, K, cfg.rope_base, rows=part),
                    np.array_split(rows, workers)))
        total = (N / len(rows)) * (time.perf_counter() - t0)
    return {"value": N / total, "unit": "rows/s", "cores": workers, "kind": "oracle",
            "sample": "%d random packed rows of %d, float64 NumPy over %d threads (each row's history, group "
                      "keys, top-k picks and attention), scaled to all rows" % (len(rows), N, workers),
            "seconds_full_estimate": total, "host_cpus": len(os.sched_getaffinity(0))}


def head_cpu_baseline(s, inp, R, n_sample=32):
    """The head-path oracle on a bounded sample: the first n_sample steps' teacher logits
    (float64 product over the whole head, in vocabulary blocks) and their E2E-TV statistics,
    scaled to all steps."""
    import numpy as np
    from oracle import e2etv_row_stats_ref, head_logits_ref, pack_ref
    from specgen import bf16_bits_to_f32

    log("timing the head oracle on %d steps" % n_sample)
    lay = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    wid = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    rows = np.arange(n_sample)
    V = inp["head"].shape[0]
    t0 = time.perf_counter()
    hidden = wid(inp["hidden"])
    y = np.empty((n_sample, V))
    for v0 in range(0, V, 16384):
        y[:, v0:v0 + 16384] = head_logits_ref(lay, hidden, wid(inp["head"][v0:v0 + 16384]), steps=rows)
    e2etv_row_stats_ref(wid(inp["draft"][:n_sample]), y)
    total = (time.perf_counter() - t0) * R / n_sample
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    return {"value": R / total, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": "the first %d of %d steps: float64 NumPy head product over the whole vocabulary "
                      "(BLAS threads) and the E2E-TV row statistics, scaled to all steps" % (n_sample, R),
            "seconds_full_estimate": total, "host_cpus": len(os.sched_getaffinity(0))}


def gdn_cpu_baseline(s, inp, C, n_rows, per_thread=2):
    """The GDN oracle on a bounded sample: features of every packed row, the whole
    trunk pass (heads split over the host threads), then the replay of per_thread
    random branches per thread from the oracle's checkpoints, scaled to all branches."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import gdn_features_ref, gdn_replay_ref, gdn_trunk_ref, pack_ref
    from specgen import bf16_bits_to_f32

    log("timing the GDN oracle on a bounded sample")
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    lay = pack_ref(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"])
    wid = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    taps = inp["taps"].astype(np.float64)
    t0 = time.perf_counter()
    q, k, v = gdn_features_ref(lay, wid(inp["xq"]), wid(inp["xk"]), wid(inp["xv"]), taps[0], taps[1], taps[2])
    t_feat = time.perf_counter() - t0
    al, be = inp["alpha"].astype(np.float64), inp["beta"].astype(np.float64)
    H = q.shape[1]
    parts = [p for p in np.array_split(np.arange(H), workers) if len(p)]
    with ThreadPoolExecutor(workers) as ex:
        t0 = time.perf_counter()
        res = list(ex.map(lambda hs: gdn_trunk_ref(lay, q[:, hs], k[:, hs], v[:, hs], al[:, hs], be[:, hs], C)[0],
                          parts))
        t_trunk = time.perf_counter() - t0
    ck = np.concatenate(res, axis=2)
    B = lay["n_branches"]
    pick = np.random.default_rng(7).choice(B, size=min(B, per_thread * workers), replace=False)
    with ThreadPoolExecutor(workers) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda part: gdn_replay_ref(lay, q, k, v, al, be, ck, C, branches=part.tolist()),
                    np.array_split(pick, workers)))
        t_rep = (B / len(pick)) * (time.perf_counter() - t0)
    total = t_feat + t_trunk + t_rep
    return {"value": n_rows / total, "unit": "rows/s", "cores": workers,
            "kind": "oracle",
            "sample": "features of all %d packed rows, the whole trunk pass, then the replay of %d random "
                      "branches of %d, float64 NumPy over %d threads; the replay scaled to all branches"
                      % (lay["n_rows"], len(pick), B, workers),
            "seconds_full_estimate": total, "host_cpus": len(os.sched_getaffinity(0))}


def ceilings(args):
    """Achievable rates on this GPU for the two roofline bounds, from the probe library
    (tree_attention_spec_amd/libspec_probe.so): HBM streams of the shapes the E2E-TV
    kernel moves (read-only, write-only, and two bf16 reads to one float32 write per
    element) with and without non-temporal loads and stores, chains of bf16 MFMAs, and
    the same MFMAs fed from LDS at the tree attention's 1 KB of fragment reads per MFMA
    (and at 1/2, 1/4 of that, and reads alone)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "tree_attention_spec_amd", "libspec_probe.so")
    if not os.path.exists(path):
        raise ImportError("libspec_probe.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    c = ctypes
    lib.spec_probe_read.argtypes = [c.c_void_p, c.c_int64, c.c_void_p, c.c_int, c.c_int, c.c_void_p]
    lib.spec_probe_write.argtypes = [c.c_void_p, c.c_int64, c.c_int, c.c_int, c.c_void_p]
    lib.spec_probe_mixed.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64, c.c_int, c.c_int, c.c_int,
                                     c.c_int, c.c_void_p]
    lib.spec_probe_mfma.argtypes = [c.c_void_p, c.c_int, c.c_int, c.c_void_p]
    lib.spec_probe_mfma_lds.argtypes = [c.c_void_p, c.c_int, c.c_int, c.c_int, c.c_void_p]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev)
    sp = c.c_void_p(stream.cuda_stream)

    def timed(fn, reps=10):
        for _ in range(2):
            assert fn() == 0
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            assert fn() == 0
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))[reps // 2]

    n = 1 << 30                          # elements of the mixed stream
    a = torch.randn(n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, device=dev).to(torch.bfloat16)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    sink = torch.zeros(16, dtype=torch.int32, device=dev)
    P = lambda t: c.c_void_p(t.data_ptr())
    res = {"device": torch.cuda.get_device_name(dev), "compute_units": cus, "streams": {}, "mfma": {}}
    grids = [0, 8 * cus, 32 * cus]
    for nt in (0, 1):
        for g in grids:
            ms = timed(lambda: lib.spec_probe_read(P(out), 4 * n, P(sink), nt, g, sp))
            res["streams"]["read nt=%d grid=%d" % (nt, g)] = {"bytes": 4 * n, "ms": ms, "GB/s": 4 * n / ms / 1e6}
            ms = timed(lambda: lib.spec_probe_write(P(out), 4 * n, nt, g, sp))
            res["streams"]["write nt=%d grid=%d" % (nt, g)] = {"bytes": 4 * n, "ms": ms, "GB/s": 4 * n / ms / 1e6}
    for ntl in (0, 1):
        for nts in (0, 1):
            for un in (1, 4):
                for g in grids:
                    ms = timed(lambda: lib.spec_probe_mixed(P(a), P(b), P(out), n, ntl, nts, un, g, sp))
                    res["streams"]["mixed bf16+bf16->f32 ntload=%d ntstore=%d unroll=%d grid=%d"
                                   % (ntl, nts, un, g)] = {"bytes": 8 * n, "ms": ms, "GB/s": 8 * n / ms / 1e6}
    # correctness of the mixed probe on a few elements (it writes a - b)
    torch.cuda.synchronize()
    idx = torch.randint(0, n, (64,), device=dev)
    assert torch.equal(out[idx], a[idx].float() - b[idx].float())
    del a, b, out
    iters = 2048
    msink = torch.zeros(cus * 8, dtype=torch.float32, device=dev)  # one float per workgroup
    for waves_per_simd in (2, 4, 8):
        blocks = cus * waves_per_simd          # 4 waves per workgroup, one per SIMD
        flop = float(blocks) * 4 * 4 * iters * 32 * 32 * 16 * 2
        ms = timed(lambda: lib.spec_probe_mfma(P(msink), blocks, iters, sp), reps=5)
        res["mfma"]["bf16 32x32x16, %d waves/SIMD" % waves_per_simd] = {"flop": flop, "ms": ms,
                                                                        "TFLOP/s": flop / ms / 1e9}
    # MFMAs fed from LDS: a fresh 1 KB A fragment every `reuse` MFMAs (1: the tree
    # attention's K and V^T fragments), or LDS reads alone (reuse 0)
    res["lds"] = {}
    iters = 4096
    for waves_per_simd in (1, 2):
        blocks = cus * waves_per_simd
        for reuse in (0, 1, 2, 4):
            lds_bytes = float(blocks) * 4 * 8 * iters * 1024
            flop = float(blocks) * 4 * 8 * iters * reuse * 32 * 32 * 16 * 2
            ms = timed(lambda: lib.spec_probe_mfma_lds(P(msink), blocks, iters, reuse, sp), reps=5)
            key = ("LDS reads only" if reuse == 0 else "bf16 32x32x16, 1 KB LDS fragment per %d MFMA" % reuse)
            res["lds"]["%s, %d waves/SIMD" % (key, waves_per_simd)] = {
                "flop": flop, "lds_bytes": lds_bytes, "ms": ms, "TFLOP/s": flop / ms / 1e9,
                "LDS GB/s": lds_bytes / ms / 1e6, "LDS B/clk/CU at 2.4 GHz": lds_bytes / (ms * 1e-3) / cus / 2.4e9}
    # a library bf16 GEMM (torch.matmul, i.e. hipBLASLt) of the fused head's product
    # shape, hidden [4096 x 4096] times head^T [4096 x 151,936]: the rate a plain
    # product of that shape reaches, for the head's roofline (operands contiguous)
    res["library_gemm"] = {}
    g = torch.Generator(device=dev).manual_seed(7)
    for (mm, kk, nn) in ((4096, 4096, 151936),):
        a = torch.randn(mm, kk, device=dev, generator=g).to(torch.bfloat16)
        b = torch.randn(kk, nn, device=dev, generator=g).to(torch.bfloat16)
        flop = 2.0 * mm * kk * nn
        ms = timed(lambda: (torch.matmul(a, b), 0)[1], reps=5)
        res["library_gemm"]["bf16 %dx%dx%d torch.matmul" % (mm, kk, nn)] = {"flop": flop, "ms": ms,
                                                                           "TFLOP/s": flop / ms / 1e9}
        del a, b
    best = lambda d, key, pre: max((v[key], k) for k, v in d.items() if k.startswith(pre))
    res["summary"] = {
        "read_GBs": best(res["streams"], "GB/s", "read"),
        "write_GBs": best(res["streams"], "GB/s", "write"),
        "mixed_GBs": best(res["streams"], "GB/s", "mixed"),
        "mfma_bf16_TFLOPs": best(res["mfma"], "TFLOP/s", "bf16"),
        "mfma_lds_1KB_per_mfma_TFLOPs": best(res["lds"], "TFLOP/s", "bf16 32x32x16, 1 KB LDS fragment per 1 "),
        "lds_read_GBs": best(res["lds"], "LDS GB/s", "LDS reads only"),
        "library_gemm_head_shape_TFLOPs": best(res["library_gemm"], "TFLOP/s", "bf16"),
        "datasheet": {"hbm_GBs": PEAK_HBM_GBS, "bf16_TFLOPs": PEAK_BF16_TFLOPS},
    }
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None,
                    help="workload (default: stress for the scoring step, gqa8b for --gdn and --head)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="also time every branch scored as its own causal sequence (uncached independent "
                         "scoring) with the same kernels, and report the ratio to the shared-prefix layout")
    ap.add_argument("--gdn", action="store_true",
                    help="time GDN scoring of the workload's tree (spec_gdn_trunk_fwd, then spec_gdn_replay_fwd) "
                         "instead of the attention + E2E-TV step, and print its own JSON line")
    ap.add_argument("--head", action="store_true",
                    help="E2E-TV from hidden states through the output head (fused readout, product, E2E-TV)")
    ap.add_argument("--qsa", action="store_true",
                    help="sparse attention with branch-consistent indexer groups (spec_qsa_attn_fwd) over the "
                         "workload's tree, with its own JSON line")
    ap.add_argument("--gdn-token-replay", action="store_true",
                    help="with --gdn: replay a token at a time instead of from the trunk pass's cache")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure achievable HBM stream and bf16 MFMA rates with the probe library and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM counters) and exit")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DB",
                    help="print per-kernel counter means from rocprofv3 --pmc databases and exit")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="write profiles/traffic.json from four rocprofv3 --pmc databases and exit")
    args = ap.parse_args()
    if args.config is None:
        args.config = "gqa8b" if (args.gdn or args.head or args.qsa) else "stress"
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc), indent=1))
        return
    if args.write_traffic:
        print(json.dumps(write_traffic(*args.write_traffic, workload=args.config), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the branch-parallel scoring path is built and timed "
              "on a single MI355X (multi-GPU sharding is a design note, not an implementation).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.ceilings:
        print(json.dumps(ceilings(args)), flush=True)
        return

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 3}), flush=True)
        return

    import tree_attention_spec_amd as tas
    from specgen import CONFIGS, gen_logit_rows, gen_logits, gen_qkv, gen_structure

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("config %s: %s" % (cfg.name, cfg.description))
    s = gen_structure(cfg)
    if args.gdn:
        print(json.dumps(gdn_bench(args, cfg, s, dev)), flush=True)
        return
    if args.head:
        print(json.dumps(head_bench(args, cfg, s, dev)), flush=True)
        return
    if args.qsa:
        print(json.dumps(qsa_bench(args, cfg, s, dev)), flush=True)
        return
    layout, mem_bytes = tas.spec_tree_pack_query(s["trunk_len"], s["n_branches"], s["anchors"],
                                                 s["branch_len"])
    N, R = layout.n_rows, layout.n_steps
    log("N=%d packed rows, R=%d supervised steps; generating inputs" % (N, R))

    def dev_tensor(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v = gen_qkv(cfg, N)
    qt, kt, vt = dev_tensor(q), dev_tensor(k), dev_tensor(v)
    z, y = gen_logits(cfg, R)
    zt, yt = dev_tensor(z), dev_tensor(y)
    del z, y
    V = cfg.vocab
    esz_logit = 2 if cfg.logit_dtype == "bf16" else 4

    mem = torch.empty(mem_bytes, dtype=torch.uint8, device=dev)
    tree = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"], mem=mem)
    out = torch.empty_like(qt)
    ro = torch.empty((R, cfg.hq, cfg.head_dim), dtype=qt.dtype, device=dev)
    awork = torch.empty(tas.attn_work_bytes(tree, cfg.hq, cfg.hkv, cfg.head_dim, qt.dtype),
                        dtype=torch.uint8, device=dev)
    alpha = torch.empty(R, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    grad = torch.empty((R, V), dtype=torch.float32, device=dev)
    ework = torch.empty(tas.e2etv_work_bytes(tree, V, zt.dtype), dtype=torch.uint8, device=dev)

    def step():
        t = tas.spec_tree_pack(s["trunk_len"], s["n_branches"], s["anchors"], s["branch_len"], mem=mem)
        tas.spec_tree_attn_fwd(t, qt, kt, vt, rope_base=cfg.rope_base, out=out, readout_out=ro, work=awork)
        tas.spec_e2etv_fwd_bwd(t, zt, yt, alpha_out=alpha, loss_out=loss, grad_out=grad, work=ework)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timers = [tas.KernelTimer(capacity=16) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        with timers[i]:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per = {}
    for tm in timers:
        for name, ms in tm.durations():
            per.setdefault(name, []).append(ms)
    avg = {n: sum(x) / len(x) for n, x in per.items()}
    log("per-kernel ms: " + ", ".join("%s %.4f" % kv for kv in avg.items()))
    log("loss %.6f, ms/step %.3f" % (loss.item(), ms_per_step))

    P = causal_pairs(s)
    attn_flop = 4.0 * cfg.head_dim * cfg.hq * P
    e2e_elems = float(R) * V
    bf16 = cfg.qkv_dtype == "bf16"
    t_attn = avg.get("tree_attn", float("nan"))
    attn_tflops = attn_flop / (t_attn * 1e-3) / 1e12
    attn_peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    e2e_kernels = [n for n in avg if n.startswith("e2etv")]
    t_e2e = sum(avg[n] for n in e2e_kernels)
    e2e_bytes = e2e_elems * (2 * esz_logit + 4)
    e2e_gbs = e2e_bytes / (t_e2e * 1e-3) / 1e9
    components = {
        "tree_attn": {"bound": "mfma", "ms": t_attn, "algorithmic_flop": attn_flop,
                      "causal_pairs": P, "achieved": attn_tflops, "peak": attn_peak,
                      "unit": "TFLOP/s", "frac": attn_tflops / attn_peak},
        "e2etv": {"bound": "hbm", "ms": t_e2e, "kernels": e2e_kernels, "algorithmic_bytes": e2e_bytes,
                  "achieved": e2e_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": e2e_gbs / PEAK_HBM_GBS},
    }
    # The dominant stage by time. E2E-TV is one operation that may span several
    # kernels (the fused pass with its clear and loss kernels, or statistics,
    # scan and gradient); its algorithmic bytes (each logit read once, the
    # gradient written once) belong to the operation, so its roofline is taken
    # over the sum of those kernels' launch durations.
    if t_attn >= t_e2e:
        roof = {"kernel": "tree_attn", "kernels": ["tree_attn"], "bound": "mfma",
                "achieved": attn_tflops, "peak": attn_peak, "unit": "TFLOP/s",
                "frac": attn_tflops / attn_peak, "algorithmic_flop_per_launch": attn_flop,
                "traffic": measured_traffic("tree_attn", source_hash(*MARK_KERNELS["tree_attn"][1]), args.config)}
    else:
        traffic = [measured_traffic(n, source_hash(*MARK_KERNELS[n][1]), args.config)
                   for n in e2e_kernels]
        roof = {"kernel": "e2etv", "kernels": e2e_kernels, "bound": "hbm", "achieved": e2e_gbs,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": e2e_gbs / PEAK_HBM_GBS,
                "algorithmic_bytes_per_launch": e2e_bytes,
                "traffic": None if any(t is None for t in traffic) else sum(traffic)}

    result = {
        "metric": "supervised rows/s (tree-attn + E2E-TV fwd/bwd)",
        "value": R / (ms_per_step * 1e-3),
        "unit": "supervised rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded; no datasets or weights)",
        "config": {"workload": cfg.name, "description": cfg.description, "n_rows": N,
                   "supervised_rows": R, "vocab": V, "heads_q": cfg.hq, "heads_kv": cfg.hkv,
                   "head_dim": cfg.head_dim, "parallelism": "single GPU"},
        "roofline": roof,
        "components": components,
        "kernel_ms": avg,
    }
    if args.ablation:
        log("ablation: every branch as its own causal sequence")
        result["ablation"] = ablation(cfg, s, tree, qt, kt, vt, out, steps=max(2, min(args.steps, 5)), warmup=2)
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(cfg, s, q, k, v, lambda rows: gen_logit_rows(cfg, R, rows), N, R)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
