"""ctypes declarations of libspec_tree.so (see include/spec_tree.h).

Loading the library requires the HIP runtime that torch already loaded, so the
package imports torch first. A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspec_tree.so")

SPEC_OK, SPEC_ERR_INVALID_ARG, SPEC_ERR_UNSUPPORTED, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP = range(5)
SPEC_F32, SPEC_BF16 = 0, 1
SPEC_MAX_BRANCH_LEN = 64

_i32p = ctypes.POINTER(ctypes.c_int32)


class spec_tree_layout(ctypes.Structure):
    _fields_ = [
        ("n_trees", ctypes.c_int32),
        ("n_branches", ctypes.c_int32),
        ("max_branch_len", ctypes.c_int32),
        ("max_pos", ctypes.c_int32),
        ("n_rows", ctypes.c_int64),
        ("n_steps", ctypes.c_int64),
        ("n_attn_items", ctypes.c_int32),
        ("max_trunk_len", ctypes.c_int32),
        ("tree_off", _i32p),
        ("tree_trunk_len", _i32p),
        ("row_tree", _i32p),
        ("row_branch", _i32p),
        ("row_anchor", _i32p),
        ("row_pos", _i32p),
        ("row_depth", _i32p),
        ("row_trunk_hi", _i32p),
        ("row_branch_lo", _i32p),
        ("branch_tree", _i32p),
        ("branch_anchor", _i32p),
        ("branch_len", _i32p),
        ("branch_off", _i32p),
        ("step_off", _i32p),
        ("branch_order", _i32p),
        ("step_branch", _i32p),
        ("step_pred_row", _i32p),
        ("step_sample_row", _i32p),
        ("attn_items", _i32p),
    ]


SPEC_PROFILE_MAX = 256


class spec_profile(ctypes.Structure):
    _fields_ = [
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("capacity", ctypes.c_int32),
        ("used", ctypes.c_int32),
        ("names", ctypes.c_char_p * SPEC_PROFILE_MAX),
    ]


# name -> (length as a function of the layout scalars)
LAYOUT_ARRAYS = {
    "tree_off": lambda L: L.n_trees + 1,
    "tree_trunk_len": lambda L: L.n_trees,
    "row_tree": lambda L: L.n_rows,
    "row_branch": lambda L: L.n_rows,
    "row_anchor": lambda L: L.n_rows,
    "row_pos": lambda L: L.n_rows,
    "row_depth": lambda L: L.n_rows,
    "row_trunk_hi": lambda L: L.n_rows,
    "row_branch_lo": lambda L: L.n_rows,
    "branch_tree": lambda L: L.n_branches,
    "branch_anchor": lambda L: L.n_branches,
    "branch_len": lambda L: L.n_branches,
    "branch_off": lambda L: L.n_branches,
    "step_off": lambda L: L.n_branches + 1,
    "branch_order": lambda L: L.n_branches,
    "step_branch": lambda L: L.n_steps,
    "step_pred_row": lambda L: L.n_steps,
    "step_sample_row": lambda L: L.n_steps,
    # the blocks, then the same blocks in groups of four ((n + 3) // 4 + 2 * n_trees groups)
    "attn_items": lambda L: (L.n_attn_items + 4 * ((L.n_attn_items + 3) // 4 + 2 * L.n_trees)) * 8,
}

EXPORTS = ["spec_tree_pack", "spec_tree_attn_fwd", "spec_e2etv_fwd_bwd", "spec_e2etv_fwd_bwd_noalloc",
           "spec_e2etv_status",
           "spec_e2etv_head_fwd_bwd", "spec_qsa_attn_fwd",
           "spec_gdn_trunk_fwd",
           "spec_gdn_replay_fwd", "spec_status_string", "spec_last_error", "spec_abi_version",
           "spec_profile_attach"]


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            "libspec_tree.so is not built (%s); run `python -m tree_attention_spec_amd.build` "
            "or __graft_entry__.build() first" % path)
    lib = ctypes.CDLL(path)
    c = ctypes
    lib.spec_tree_pack.restype = c.c_int
    lib.spec_tree_pack.argtypes = [c.c_int32, _i32p, _i32p, _i32p, _i32p, c.c_void_p,
                                   c.POINTER(c.c_size_t), c.POINTER(spec_tree_layout), c.c_void_p]
    lib.spec_tree_attn_fwd.restype = c.c_int
    lib.spec_tree_attn_fwd.argtypes = [c.POINTER(spec_tree_layout), c.c_int32, c.c_int32, c.c_int32,
                                       c.c_int, c.c_void_p, c.c_void_p, c.c_void_p, c.c_float,
                                       c.c_float, c.c_void_p, c.c_void_p, c.c_void_p,
                                       c.POINTER(c.c_size_t), c.c_void_p]
    lib.spec_e2etv_fwd_bwd.restype = c.c_int
    lib.spec_e2etv_fwd_bwd.argtypes = [c.POINTER(spec_tree_layout), c.c_int64, c.c_int, c.c_void_p,
                                       c.c_void_p, c.c_float, c.c_void_p, c.c_void_p, c.c_void_p,
                                       c.c_void_p, c.POINTER(c.c_size_t), c.c_void_p]
    lib.spec_e2etv_fwd_bwd_noalloc.restype = c.c_int
    lib.spec_e2etv_fwd_bwd_noalloc.argtypes = [c.POINTER(spec_tree_layout), c.c_int64, c.c_int, c.c_void_p,
                                               c.c_void_p, c.c_float, c.c_void_p, c.c_void_p, c.c_void_p,
                                               c.c_void_p]
    lib.spec_e2etv_status.restype = c.c_int
    lib.spec_e2etv_status.argtypes = [c.POINTER(spec_tree_layout), c.c_int64, c.c_void_p,
                                      c.POINTER(c.c_uint32), c.c_void_p]
    lib.spec_qsa_attn_fwd.restype = c.c_int
    lib.spec_qsa_attn_fwd.argtypes = [c.POINTER(spec_tree_layout), c.c_int32, c.c_int32, c.c_int32, c.c_int32,
                                      c.c_int32, c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                      c.c_void_p, c.c_float, c.c_float, c.c_void_p, c.c_void_p, c.c_void_p,
                                      c.c_void_p, c.POINTER(c.c_size_t), c.c_void_p]
    lib.spec_e2etv_head_fwd_bwd.restype = c.c_int
    lib.spec_e2etv_head_fwd_bwd.argtypes = [c.POINTER(spec_tree_layout), c.c_int64, c.c_int32,
                                            c.c_int, c.c_void_p, c.c_void_p, c.c_void_p, c.c_float,
                                            c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                            c.POINTER(c.c_size_t), c.c_void_p]
    lib.spec_gdn_trunk_fwd.restype = c.c_int
    lib.spec_gdn_trunk_fwd.argtypes = [c.POINTER(spec_tree_layout), c.c_int32, c.c_int32, c.c_int32,
                                       c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                       c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                       c.POINTER(c.c_size_t), c.c_void_p]
    lib.spec_gdn_replay_fwd.restype = c.c_int
    lib.spec_gdn_replay_fwd.argtypes = [c.POINTER(spec_tree_layout), c.c_int32, c.c_int32, c.c_int32,
                                        c.c_int32, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                        c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                        c.c_void_p]
    lib.spec_status_string.restype = c.c_char_p
    lib.spec_status_string.argtypes = [c.c_int]
    lib.spec_last_error.restype = c.c_char_p
    lib.spec_last_error.argtypes = []
    lib.spec_abi_version.restype = c.c_int32
    lib.spec_abi_version.argtypes = []
    lib.spec_profile_attach.restype = None
    lib.spec_profile_attach.argtypes = [c.POINTER(spec_profile)]
    return lib


class SpecError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, status), message))
        self.status = status


_STATUS_NAMES = {SPEC_OK: "SPEC_OK", SPEC_ERR_INVALID_ARG: "SPEC_ERR_INVALID_ARG",
                 SPEC_ERR_UNSUPPORTED: "SPEC_ERR_UNSUPPORTED",
                 SPEC_ERR_WORKSPACE: "SPEC_ERR_WORKSPACE", SPEC_ERR_HIP: "SPEC_ERR_HIP"}


def check(lib: ctypes.CDLL, status: int):
    if status != SPEC_OK:
        raise SpecError(status, lib.spec_last_error().decode(errors="replace"))
