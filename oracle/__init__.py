"""CPU oracle for the branch-parallel scoring path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy float64 statement of what the path
computes: the proposal-tree pack, tree-masked GQA attention with RoPE at
semantic positions, predecessor-row readout, the E2E-TV surrogate with its
gradient (also with teacher logits formed through an output head), indexed GDN state replay for
linear-attention targets, and sparse attention with branch-consistent indexer groups. It shares no code with the HIP library and imports nothing from it;
the only shared module is ``specgen`` (seeded inputs, no method arithmetic).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path never calls it.

Sources, cited by page title and section throughout:
  * [SpecOPD paper page] "SpecOPD: Branch-Parallel On-Policy Distillation for
    Speculative Decoding" (thelatestinai.com paper page): abstract and the
    captions of Figures 2, 3, 4, 5 and 13.
  * [SpecOPD notes page] "SpecOPD: independent supervision branches and
    acceptance-prefix optimization" (daiwk auto-research notes): sections
    "Equations", "Inputs and code mapping" and "Checks, negative controls,
    and limits".

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (a hand-worked example, a closed form, brute force, a library
routine or finite differences); none is "parity unpinned".
"""
from .pack_ref import pack_ref, parents_ref, visible_ref, visible_intervals_ref  # noqa: F401
from .attn_ref import (  # noqa: F401
    brute_force_branch_ref,
    causal_attn_ref,
    readout_ref,
    rope_ref,
    tree_attn_ref,
)
from .e2etv_ref import (  # noqa: F401
    e2etv_coef_ref,
    e2etv_grad_ref,
    e2etv_loss_ref,
    e2etv_ref,
    e2etv_row_stats_ref,
)
from .head_ref import e2etv_head_ref, head_logits_ref  # noqa: F401
from .qsa_ref import (  # noqa: F401
    qsa_attn_ref,
    qsa_brute_force_branch_ref,
    qsa_causal_ref,
    qsa_group_keys,
    qsa_history_ref,
    qsa_pick,
    qsa_row_structure,
)
from .gdn_ref import (  # noqa: F401
    ancestors_ref,
    conv_ancestry_ref,
    gdn_branch_brute_ref,
    gdn_checkpoints_ref,
    gdn_trunk_ref,
    gdn_features_ref,
    gdn_replay_ref,
    gdn_step_ref,
    silu,
    trunk_len_ref,
)
