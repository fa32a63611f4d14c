"""Branch-parallel scoring path on MI355X: Python binding of libspec_tree.so.

The three calls mirror the C ABI in ``include/spec_tree.h`` and do argument
marshalling only: torch provides device memory and the current HIP stream,
every step of the path runs in the library's HIP kernels.

    tree = spec_tree_pack(trunk_len, n_branches, anchors, branch_len, device="cuda")
    out, readout = spec_tree_attn_fwd(tree, q, k, v, rope_base=10000.0)
    alpha, loss, grad = spec_e2etv_fwd_bwd(tree, draft_logits, teacher_logits)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # loads the HIP runtime the library binds to; keep before the library

from . import _lib
from ._lib import (LAYOUT_ARRAYS, SPEC_BF16, SPEC_F32, SPEC_MAX_BRANCH_LEN, SpecError,  # noqa: F401
                   spec_tree_layout)

__all__ = ["spec_tree_pack", "spec_tree_pack_query", "spec_tree_attn_fwd", "spec_e2etv_fwd_bwd",
           "spec_e2etv_head_fwd_bwd", "e2etv_head_work_bytes", "spec_qsa_attn_fwd", "qsa_work_bytes",
           "spec_e2etv_fwd_bwd_noalloc", "spec_e2etv_status",
           "spec_gdn_trunk_fwd", "spec_gdn_replay_fwd", "gdn_checkpoint_slots", "gdn_trunk_work_bytes", "PackedTree", "SpecError", "library",
           "KernelTimer"]

_LIB = None


def library() -> ctypes.CDLL:
    """The loaded libspec_tree.so (raises ImportError if it is not built). The
    SPEC_TREE_LIBRARY environment variable names another build of the same library
    (the CPU tests use it for the host-sanitized build)."""
    global _LIB
    if _LIB is None:
        _LIB = _lib.load(os.environ.get("SPEC_TREE_LIBRARY") or _lib.LIB_PATH)
    return _LIB


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64).astype(np.int32))


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if a.size else None


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError("tensors must be bfloat16 or float32, got %s" % t.dtype)


class PackedTree:
    """A packed proposal tree: the layout struct plus the device buffer it points into."""

    def __init__(self, layout: spec_tree_layout, mem: torch.Tensor):
        self.layout = layout
        self.mem = mem

    n_trees = property(lambda s: s.layout.n_trees)
    n_branches = property(lambda s: s.layout.n_branches)
    n_rows = property(lambda s: s.layout.n_rows)
    n_steps = property(lambda s: s.layout.n_steps)
    max_branch_len = property(lambda s: s.layout.max_branch_len)
    max_pos = property(lambda s: s.layout.max_pos)
    n_attn_items = property(lambda s: s.layout.n_attn_items)
    max_trunk_len = property(lambda s: s.layout.max_trunk_len)
    device = property(lambda s: s.mem.device)

    def arrays(self) -> dict:
        """Device int32 views of every layout array, by name."""
        base = self.mem.data_ptr()
        words = self.mem.view(torch.int32)
        out = {}
        for name, length in LAYOUT_ARRAYS.items():
            ptr = ctypes.cast(getattr(self.layout, name), ctypes.c_void_p).value
            n = int(length(self.layout))
            if ptr is None or n == 0:
                out[name] = torch.zeros(0, dtype=torch.int32, device=self.mem.device)
                continue
            off = (ptr - base) // 4
            out[name] = words[off:off + n]
        return out


def spec_tree_pack_query(trunk_len, n_branches, anchors, branch_len):
    """Size query (no GPU work): returns (layout scalars, bytes of the device buffer)."""
    lib = library()
    T, nb, a, w = _i32(trunk_len), _i32(n_branches), _i32(anchors), _i32(branch_len)
    layout = spec_tree_layout()
    nbytes = ctypes.c_size_t(0)
    _lib.check(lib, lib.spec_tree_pack(len(T), _iptr(T), _iptr(nb), _iptr(a), _iptr(w), None,
                                       ctypes.byref(nbytes), ctypes.byref(layout), None))
    return layout, nbytes.value


def spec_tree_pack(trunk_len, n_branches, anchors, branch_len, device=None, mem=None) -> PackedTree:
    """Pack proposal trees on ``device``; ``mem`` may supply a reusable uint8 buffer."""
    lib = library()
    device = torch.device(device if device is not None else "cuda")
    T, nb, a, w = _i32(trunk_len), _i32(n_branches), _i32(anchors), _i32(branch_len)
    if mem is None:
        _, need = spec_tree_pack_query(T, nb, a, w)
        mem = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    layout = spec_tree_layout()
    nbytes = ctypes.c_size_t(mem.numel())
    call = lambda m: lib.spec_tree_pack(len(T), _iptr(T), _iptr(nb), _iptr(a), _iptr(w),
                                        ctypes.c_void_p(m.data_ptr()), ctypes.byref(nbytes),
                                        ctypes.byref(layout), ctypes.c_void_p(_stream(device)))
    st = call(mem)
    if st == _lib.SPEC_ERR_WORKSPACE:          # buffer too small: nbytes now holds the need
        mem = torch.empty(nbytes.value, dtype=torch.uint8, device=device)
        st = call(mem)
    _lib.check(lib, st)
    return PackedTree(layout, mem)


def _attn_call(tree, hq, hkv, D, dt, q, k, v, rope_base, scale, out, readout, work):
    lib = library()
    nbytes = ctypes.c_size_t(work.numel() if work is not None else 0)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    return lib.spec_tree_attn_fwd(ctypes.byref(tree.layout), hq, hkv, D, dt, ptr(q), ptr(k), ptr(v),
                                  float(rope_base), float(scale), ptr(out), ptr(readout), ptr(work),
                                  ctypes.byref(nbytes),
                                  ctypes.c_void_p(_stream(q.device)) if q is not None else None), nbytes.value


def attn_work_bytes(tree, n_heads_q, n_heads_kv, head_dim, dtype) -> int:
    lib = library()
    nbytes = ctypes.c_size_t(0)
    dt = SPEC_BF16 if dtype == torch.bfloat16 else SPEC_F32
    _lib.check(lib, lib.spec_tree_attn_fwd(ctypes.byref(tree.layout), n_heads_q, n_heads_kv, head_dim,
                                           dt, None, None, None, 10000.0, 0.0, None, None, None,
                                           ctypes.byref(nbytes), None))
    return nbytes.value


def spec_tree_attn_fwd(tree: PackedTree, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       rope_base: float = 10000.0, softmax_scale: float = 0.0, readout: bool = True,
                       out: torch.Tensor = None, readout_out: torch.Tensor = None,
                       work: torch.Tensor = None):
    """Tree attention. q [N,Hq,D], k/v [N,Hkv,D] (bf16 or fp32, contiguous, on the GPU).

    Returns (out [N,Hq,D], readout [R,Hq,D] or None).
    """
    N, hq, D = q.shape
    hkv = k.shape[1]
    if k.shape != (N, hkv, D) or v.shape != (N, hkv, D) or N != tree.n_rows:
        raise ValueError("q/k/v shapes do not match the packed tree")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k and v must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if readout and readout_out is None:
        readout_out = torch.empty((tree.n_steps, hq, D), dtype=q.dtype, device=q.device)
    if not readout:
        readout_out = None
    if work is None:
        work = torch.empty(max(attn_work_bytes(tree, hq, hkv, D, q.dtype), 256), dtype=torch.uint8,
                           device=q.device)
    st, _ = _attn_call(tree, hq, hkv, D, dt, q, k, v, rope_base, softmax_scale, out, readout_out, work)
    _lib.check(library(), st)
    return out, readout_out


def _qsa_call(tree, hq, hkv, D, di, G, top_k, q, k, v, qi, ki, rope_base, scale, out, sel, readout, work):
    lib = library()
    nbytes = ctypes.c_size_t(work.numel() if work is not None else 0)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    dev = q.device if q is not None else None
    return lib.spec_qsa_attn_fwd(ctypes.byref(tree.layout), hq, hkv, D, di, G, top_k, ptr(q), ptr(k), ptr(v),
                                 ptr(qi), ptr(ki), float(rope_base), float(scale), ptr(out), ptr(sel),
                                 ptr(readout), ptr(work), ctypes.byref(nbytes),
                                 ctypes.c_void_p(_stream(dev)) if dev is not None else None), nbytes.value


def qsa_work_bytes(tree, n_heads_q, n_heads_kv, head_dim, index_dim, group_size, top_k) -> int:
    st, n = _qsa_call(tree, n_heads_q, n_heads_kv, head_dim, index_dim, group_size, top_k, None, None, None,
                      None, None, 10000.0, 0.0, None, None, None, None)
    _lib.check(library(), st)
    return n


def spec_qsa_attn_fwd(tree: PackedTree, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      qi: torch.Tensor, ki: torch.Tensor, group_size: int, top_k: int,
                      rope_base: float = 10000.0, softmax_scale: float = 0.0, out=None, selected=None,
                      readout: bool = True, readout_out=None, work=None):
    """Sparse attention with branch-consistent indexer groups over a packed tree.

    q [N, Hq, 128], k / v [N, Hkv, 128], qi / ki [N, Hkv, DI], all bf16. Returns
    (out [N, Hq, 128] bf16, selected [N, Hkv, top_k] int32 ascending group indices
    with -1 padding, readout [R, Hq, 128] bf16 or None)."""
    N, hq, D = q.shape
    hkv, di = ki.shape[1], ki.shape[2]
    if N != tree.n_rows or k.shape != (N, hkv, D) or v.shape != (N, hkv, D) or qi.shape != (N, hkv, di):
        raise ValueError("q [N,Hq,D], k/v [N,Hkv,D], qi/ki [N,Hkv,DI] with N = tree.n_rows")
    for t in (q, k, v, qi, ki):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("sparse attention inputs must be contiguous bf16")
    if out is None:
        out = torch.empty_like(q)
    if selected is None:
        selected = torch.empty((N, hkv, top_k), dtype=torch.int32, device=q.device)
    if readout and readout_out is None and tree.n_steps > 0:
        readout_out = torch.empty((tree.n_steps, hq, D), dtype=q.dtype, device=q.device)
    if not readout:
        readout_out = None
    if work is None:
        work = torch.empty(max(qsa_work_bytes(tree, hq, hkv, D, di, group_size, top_k), 256), dtype=torch.uint8,
                           device=q.device)
    st, _ = _qsa_call(tree, hq, hkv, D, di, group_size, top_k, q, k, v, qi, ki, rope_base, softmax_scale, out,
                      selected, readout_out, work)
    _lib.check(library(), st)
    return out, selected, readout_out


def e2etv_work_bytes(tree, vocab, dtype) -> int:
    lib = library()
    nbytes = ctypes.c_size_t(0)
    dt = SPEC_BF16 if dtype == torch.bfloat16 else SPEC_F32
    _lib.check(lib, lib.spec_e2etv_fwd_bwd(ctypes.byref(tree.layout), vocab, dt, None, None, 0.0,
                                           None, None, None, None, ctypes.byref(nbytes), None))
    return nbytes.value


def spec_e2etv_fwd_bwd(tree: PackedTree, draft: torch.Tensor, teacher: torch.Tensor,
                       inv_norm: float = 0.0, grad: bool = True, alpha_out=None, loss_out=None,
                       grad_out=None, work: torch.Tensor = None):
    """E2E-TV over logits [R, V]. Returns (alpha [R] fp32, loss [1] fp32, grad [R,V] fp32 or None)."""
    R, V = draft.shape
    if teacher.shape != (R, V) or R != tree.n_steps:
        raise ValueError("draft/teacher must be [n_steps, vocab]")
    if not (draft.is_contiguous() and teacher.is_contiguous()) or draft.dtype != teacher.dtype:
        raise ValueError("draft and teacher must be contiguous and share a dtype")
    dt = _dtype_code(draft)
    dev = draft.device
    if alpha_out is None:
        alpha_out = torch.empty(R, dtype=torch.float32, device=dev)
    if loss_out is None:
        loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    if grad and grad_out is None:
        grad_out = torch.empty((R, V), dtype=torch.float32, device=dev)
    if not grad:
        grad_out = None
    if work is None:
        work = torch.empty(max(e2etv_work_bytes(tree, V, draft.dtype), 256), dtype=torch.uint8,
                           device=dev)
    lib = library()
    nbytes = ctypes.c_size_t(work.numel())
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    _lib.check(lib, lib.spec_e2etv_fwd_bwd(ctypes.byref(tree.layout), V, dt, ptr(draft), ptr(teacher),
                                           float(inv_norm), ptr(alpha_out), ptr(loss_out),
                                           ptr(grad_out), ptr(work), ctypes.byref(nbytes),
                                           ctypes.c_void_p(_stream(dev))))
    return alpha_out, loss_out, grad_out


def spec_e2etv_status(tree: PackedTree, vocab: int, work=None, device=None) -> int:
    """Status word of the last E2E-TV call on `work` (None: the no-allocation array of the
    current device), after waiting for the current stream: 0 when every bounded wait of
    the team kernels was met."""
    lib = library()
    v = ctypes.c_uint32(0)
    dev = work.device if work is not None else (device or torch.device("cuda", torch.cuda.current_device()))
    _lib.check(lib, lib.spec_e2etv_status(ctypes.byref(tree.layout), int(vocab),
                                          ctypes.c_void_p(work.data_ptr()) if work is not None else None,
                                          ctypes.byref(v), ctypes.c_void_p(_stream(dev))))
    return v.value


def spec_e2etv_fwd_bwd_noalloc(tree: PackedTree, draft: torch.Tensor, teacher: torch.Tensor,
                               inv_norm: float = 0.0, alpha_out=None, loss_out=None, grad_out=None):
    """spec_e2etv_fwd_bwd with the library's own per-GPU workspace: the call allocates
    nothing itself, so every output tensor must be passed in (grad_out may be None for a
    forward-only call). Returns (alpha_out, loss_out, grad_out)."""
    R, V = draft.shape
    if teacher.shape != (R, V) or R != tree.n_steps:
        raise ValueError("draft/teacher must be [n_steps, vocab]")
    if not (draft.is_contiguous() and teacher.is_contiguous()) or draft.dtype != teacher.dtype:
        raise ValueError("draft and teacher must be contiguous and share a dtype")
    if alpha_out is None or loss_out is None:
        raise ValueError("the no-allocation call needs alpha_out and loss_out")
    lib = library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    _lib.check(lib, lib.spec_e2etv_fwd_bwd_noalloc(ctypes.byref(tree.layout), V, _dtype_code(draft),
                                                   ptr(draft), ptr(teacher), float(inv_norm),
                                                   ptr(alpha_out), ptr(loss_out), ptr(grad_out),
                                                   ctypes.c_void_p(_stream(draft.device))))
    return alpha_out, loss_out, grad_out


def e2etv_head_work_bytes(tree, vocab, d_model, draft_dtype=torch.bfloat16) -> int:
    lib = library()
    nbytes = ctypes.c_size_t(0)
    dt = SPEC_BF16 if draft_dtype == torch.bfloat16 else SPEC_F32
    _lib.check(lib, lib.spec_e2etv_head_fwd_bwd(ctypes.byref(tree.layout), vocab, d_model, dt, None,
                                                None, None, 0.0, None, None, None, None,
                                                ctypes.byref(nbytes), None))
    return nbytes.value


def spec_e2etv_head_fwd_bwd(tree: PackedTree, draft: torch.Tensor, hidden: torch.Tensor,
                            head: torch.Tensor, inv_norm: float = 0.0, grad: bool = True,
                            alpha_out=None, loss_out=None, grad_out=None, work: torch.Tensor = None):
    """E2E-TV with teacher logits hidden[step_pred_row] @ head^T formed on the device and never
    stored. draft [R, V] (bf16 or fp32), hidden [N, d] bf16, head [V, d] bf16.
    Returns (alpha [R] fp32, loss [1] fp32, grad [R, V] fp32 or None)."""
    R, V = draft.shape
    if R != tree.n_steps or head.dim() != 2 or head.shape[0] != V:
        raise ValueError("draft must be [n_steps, vocab] and head [vocab, d_model]")
    d = head.shape[1]
    if hidden.shape != (tree.n_rows, d):
        raise ValueError("hidden must be [n_rows, d_model]")
    if hidden.dtype != torch.bfloat16 or head.dtype != torch.bfloat16:
        raise ValueError("hidden and head must be bfloat16")
    if not (draft.is_contiguous() and hidden.is_contiguous() and head.is_contiguous()):
        raise ValueError("draft, hidden and head must be contiguous")
    dt = _dtype_code(draft)
    dev = draft.device
    if alpha_out is None:
        alpha_out = torch.empty(R, dtype=torch.float32, device=dev)
    if loss_out is None:
        loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    if grad and grad_out is None:
        grad_out = torch.empty((R, V), dtype=torch.float32, device=dev)
    if not grad:
        grad_out = None
    if work is None:
        work = torch.empty(max(e2etv_head_work_bytes(tree, V, d, draft.dtype), 256),
                           dtype=torch.uint8, device=dev)
    lib = library()
    nbytes = ctypes.c_size_t(work.numel())
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    _lib.check(lib, lib.spec_e2etv_head_fwd_bwd(ctypes.byref(tree.layout), V, d, dt, ptr(draft),
                                                ptr(hidden), ptr(head), float(inv_norm),
                                                ptr(alpha_out), ptr(loss_out), ptr(grad_out),
                                                ptr(work), ctypes.byref(nbytes),
                                                ctypes.c_void_p(_stream(dev))))
    return alpha_out, loss_out, grad_out


def gdn_checkpoint_slots(tree: PackedTree, chunk: int) -> int:
    """Checkpoint slots per tree that spec_gdn_replay_fwd indexes: max_trunk_len // chunk + 1."""
    return tree.max_trunk_len // chunk + 1


def gdn_trunk_work_bytes(tree: PackedTree, n_heads: int, head_dim: int, conv_width: int,
                         chunk: int) -> int:
    """Bytes of the workspace spec_gdn_trunk_fwd needs (a size query; no GPU work)."""
    lib = library()
    n = ctypes.c_size_t(0)
    _lib.check(lib, lib.spec_gdn_trunk_fwd(ctypes.byref(tree.layout), n_heads, head_dim, conv_width,
                                           chunk, None, None, None, None, None, None, None, None, None,
                                           ctypes.byref(n), None))
    return n.value


def _check_gdn(tree, xq, xk, xv, taps, alpha, beta, chunk):
    N, H, D = xq.shape
    if xk.shape != (N, H, D) or xv.shape != (N, H, D) or N != tree.n_rows:
        raise ValueError("xq/xk/xv must be [n_rows, H, D]")
    if not (xq.dtype == xk.dtype == xv.dtype == torch.bfloat16):
        raise TypeError("xq, xk and xv must be bfloat16")
    K = taps.shape[-1]
    if taps.shape != (3, H, D, K) or taps.dtype != torch.float32:
        raise ValueError("taps must be float32 [3, H, D, K]")
    if alpha.shape != (N, H) or beta.shape != (N, H) or alpha.dtype != torch.float32 \
            or beta.dtype != torch.float32:
        raise ValueError("alpha and beta must be float32 [n_rows, H]")
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    for t in (xq, xk, xv, taps, alpha, beta):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    return N, H, D, K, (tree.n_trees, gdn_checkpoint_slots(tree, chunk), H, D, D)


def spec_gdn_trunk_fwd(tree: PackedTree, xq: torch.Tensor, xk: torch.Tensor, xv: torch.Tensor,
                       taps: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor, chunk: int = 64,
                       ckpt: torch.Tensor = None, out: torch.Tensor = None, work: torch.Tensor = None):
    """Shared GDN trunk pass: every trunk row's output and the checkpoints.

    Inputs as for spec_gdn_replay_fwd. Returns (ckpt, out): ckpt [n_trees, slots,
    H, D, D] fp32 key-major, slot c of tree t the state after its first c*chunk
    trunk tokens (slots past floor(T_t / chunk) as passed in, zero for a new
    tensor); out [N,H,D] fp32 with the trunk rows written (branch rows as passed
    in, zero for a new tensor). ``work`` is an optional uint8 device workspace
    reused across calls (allocated when missing or too small).
    """
    N, H, D, K, ck_shape = _check_gdn(tree, xq, xk, xv, taps, alpha, beta, chunk)
    if ckpt is None:
        ckpt = torch.zeros(ck_shape, dtype=torch.float32, device=xq.device)
    elif ckpt.shape != ck_shape or ckpt.dtype != torch.float32 or not ckpt.is_contiguous():
        raise ValueError("ckpt must be contiguous float32 %s" % (list(ck_shape),))
    if out is None:
        out = torch.zeros((N, H, D), dtype=torch.float32, device=xq.device)
    lib = library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    nbytes = ctypes.c_size_t(gdn_trunk_work_bytes(tree, H, D, K, chunk))
    if work is None or work.numel() < nbytes.value:
        work = torch.empty(nbytes.value, dtype=torch.uint8, device=xq.device)
    elif work.device != xq.device or not work.is_contiguous():
        raise ValueError("work must be a contiguous tensor on the inputs' device")
    st = lib.spec_gdn_trunk_fwd(ctypes.byref(tree.layout), H, D, K, chunk, ptr(xq), ptr(xk), ptr(xv),
                                ptr(taps), ptr(alpha), ptr(beta), ptr(ckpt), ptr(out), ptr(work),
                                ctypes.byref(nbytes), ctypes.c_void_p(_stream(xq.device)))
    _lib.check(lib, st)
    return ckpt, out


def spec_gdn_replay_fwd(tree: PackedTree, xq: torch.Tensor, xk: torch.Tensor, xv: torch.Tensor,
                        taps: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                        ckpt: torch.Tensor, chunk: int = 64, out: torch.Tensor = None,
                        trunk_work: torch.Tensor = None):
    """Indexed GDN state replay for the branch rows.

    xq/xk/xv [N,H,D] bf16, taps [3,H,D,K] fp32, alpha/beta [N,H] fp32, ckpt
    [n_trees, slots, H, D, D] fp32 (key-major states, slots = gdn_checkpoint_slots,
    as spec_gdn_trunk_fwd writes them). ``trunk_work``: the workspace of the
    spec_gdn_trunk_fwd call that wrote ``ckpt`` (chunk <= 64), unchanged since;
    the replay then runs a chunk at a time from its cache. Without it the replay
    walks the tokens one at a time. Returns out [N,H,D] fp32 with the branch rows
    written (trunk rows as passed in, zero for a new tensor).
    """
    N, H, D, K, ck_shape = _check_gdn(tree, xq, xk, xv, taps, alpha, beta, chunk)
    if ckpt.shape != ck_shape or ckpt.dtype != torch.float32 or not ckpt.is_contiguous():
        raise ValueError("ckpt must be contiguous float32 %s" % (list(ck_shape),))
    if out is None:
        out = torch.zeros((N, H, D), dtype=torch.float32, device=xq.device)
    lib = library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    if trunk_work is not None and (trunk_work.device != xq.device or not trunk_work.is_contiguous()):
        raise ValueError("trunk_work must be a contiguous tensor on the inputs' device")
    st = lib.spec_gdn_replay_fwd(ctypes.byref(tree.layout), H, D, K, chunk, ptr(xq), ptr(xk), ptr(xv),
                                 ptr(taps), ptr(alpha), ptr(beta), ptr(ckpt),
                                 None if trunk_work is None else ptr(trunk_work), ptr(out),
                                 ctypes.c_void_p(_stream(xq.device)))
    _lib.check(lib, st)
    return out


class KernelTimer:
    """Per-kernel HIP-event timing of library calls on this thread (measurement only).

    While attached, each call records an event before its first kernel and after
    every kernel on the stream it launches on; ``durations()`` returns
    (kernel name, milliseconds) pairs in launch order.
    """

    def __init__(self, capacity: int = _lib.SPEC_PROFILE_MAX):
        self.capacity = min(capacity, _lib.SPEC_PROFILE_MAX)
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(self.capacity)]
        for e in self.events:          # torch creates the HIP event on first record
            e.record()
        torch.cuda.synchronize()
        self._handles = (ctypes.c_void_p * self.capacity)(*[e.cuda_event for e in self.events])
        self.prof = _lib.spec_profile()
        self.prof.events = ctypes.cast(self._handles, ctypes.POINTER(ctypes.c_void_p))
        self.prof.capacity = self.capacity

    def __enter__(self):
        self.prof.used = 0
        library().spec_profile_attach(ctypes.byref(self.prof))
        return self

    def __exit__(self, *exc):
        library().spec_profile_attach(None)

    def durations(self):
        torch.cuda.synchronize()
        out = []
        for i in range(1, self.prof.used):
            name = self.prof.names[i].decode()
            if name.endswith(":begin"):
                continue
            out.append((name, self.events[i - 1].elapsed_time(self.events[i])))
        return out
