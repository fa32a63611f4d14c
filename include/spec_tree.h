/*
 * spec_tree.h -- C ABI of the branch-parallel scoring path (MI355X / gfx950).
 *
 * Three calls make up the path, each enqueued on the caller's HIP stream:
 *   spec_tree_pack      proposal-tree packer (host checks + device expand)
 *   spec_tree_attn_fwd  tree-masked GQA attention, RoPE at semantic positions,
 *                       optional predecessor-row readout
 *   spec_e2etv_fwd_bwd  E2E-TV overlap, prefix-product loss and its gradient
 *                       with respect to the draft logits
 * Beside them:
 *   spec_e2etv_fwd_bwd_noalloc  the same E2E-TV call with a library-owned
 *                       workspace, for callers that cannot allocate
 *   spec_e2etv_head_fwd_bwd  E2E-TV with the teacher logits formed through an
 *                       output head from hidden states (never stored)
 *   spec_gdn_trunk_fwd, spec_gdn_replay_fwd  GDN scoring for linear-attention
 *                       targets: shared trunk pass, indexed state replay
 *   spec_qsa_attn_fwd   sparse attention with branch-consistent indexer groups
 *
 * Sources, cited by page title and section:
 *   [SpecOPD paper page]  "SpecOPD: Branch-Parallel On-Policy Distillation for
 *                         Speculative Decoding" (thelatestinai.com paper page)
 *   [SpecOPD notes page]  "SpecOPD: independent supervision branches and
 *                         acceptance-prefix optimization" (daiwk auto-research
 *                         notes)
 *
 * Conventions shared by every call
 *   - All pointers named d_* are device pointers; h_* are host pointers.
 *   - The caller allocates and owns every buffer. The library never allocates
 *     or frees device memory; scratch memory comes from a caller workspace
 *     (spec_e2etv_fwd_bwd_noalloc alone uses a fixed device array the loaded
 *     library holds per GPU instead).
 *     Passing d_mem / d_work == NULL is a size query: the call validates what
 *     it can, writes the byte count and returns SPEC_OK without touching the
 *     GPU (no HIP call at all).
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream). There is no host synchronisation inside any call
 *     except that spec_tree_pack's small host-to-device copy reads its host
 *     staging before returning. Device buffers must stay valid until the
 *     enqueued work completes.
 *   - Arguments are checked before anything is enqueued; on any error nothing
 *     is launched and spec_last_error() describes the problem (thread-local).
 *   - Tensors are dense and row-major. Device buffers must be 16-byte aligned.
 *   - The library holds no state between calls; calls on different streams
 *     may run concurrently as long as their buffers are disjoint (calls of
 *     spec_e2etv_fwd_bwd_noalloc on one GPU share its array and must not).
 */
#ifndef SPEC_TREE_H
#define SPEC_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_TREE_ABI_VERSION 7
#define SPEC_MAX_BRANCH_LEN 64 /* largest supported branch width W_b */

typedef enum spec_status {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARG = 1, /* a NULL / misaligned pointer or an out-of-range value */
  SPEC_ERR_UNSUPPORTED = 2, /* a valid request outside what the kernels implement */
  SPEC_ERR_WORKSPACE = 3,   /* the workspace / layout buffer is too small */
  SPEC_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} spec_status;

/* Callers may pass any 32-bit value as a spec_dtype (the library refuses the
 * ones it does not know): the two range markers make every int32 a value of the
 * enumeration, so an unknown code is an error return and never undefined. */
typedef enum spec_dtype {
  SPEC_F32 = 0,  /* IEEE binary32 */
  SPEC_BF16 = 1, /* bfloat16 (upper half of a binary32) */
  SPEC_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  SPEC_DTYPE_RANGE_MAX_ = 2147483647
} spec_dtype;

typedef void *spec_stream; /* a hipStream_t */

/*
 * Packed proposal-tree layout, filled by spec_tree_pack.
 *
 * Packed order (rows and columns of the tree mask share it, [SpecOPD paper
 * page, Figure 3]): tree by tree; inside a tree the trunk rows 0..T-1 first,
 * then the tree's branches in ascending anchor order (ties keep the caller's
 * order), each branch's rows y_{b,1}..y_{b,W_b-1} in depth order. The terminal
 * sample y_{b,W_b} has no row ([SpecOPD paper page, Figure 3]: terminal
 * samples use predecessor readouts and need no query rows), so
 *   N = n_rows  = sum_t T_t + sum_b (W_b - 1)
 *   R = n_steps = sum_b W_b   (supervised steps = E2E-TV rows).
 * Supervised steps stay in caller branch order: branch b's steps are
 * step_off[b] .. step_off[b+1]-1, step i (1-based) at step_off[b] + i - 1.
 *
 * Every device pointer points into the caller's d_mem buffer; all arrays are
 * int32. "local" anchors are zero-based trunk indices of the branch's tree
 * ([SpecOPD notes page, "Inputs and code mapping"]).
 */
typedef struct spec_tree_layout {
  /* host scalars */
  int32_t n_trees;
  int32_t n_branches;      /* B */
  int32_t max_branch_len;  /* max_b W_b (0 when B == 0) */
  int32_t max_pos;         /* largest semantic position of any row */
  int64_t n_rows;          /* N */
  int64_t n_steps;         /* R */
  int32_t n_attn_items;    /* query blocks in attn_items */
  int32_t max_trunk_len;   /* largest trunk length T_t */

  /* per tree */
  int32_t *tree_off;        /* [n_trees+1] first packed row of each tree; last = N */
  int32_t *tree_trunk_len;  /* [n_trees] trunk length T_t */
  /* per packed row [N] */
  int32_t *row_tree;        /* tree index */
  int32_t *row_branch;      /* branch index b, -1 for trunk rows */
  int32_t *row_anchor;      /* local anchor a_b, -1 for trunk rows */
  int32_t *row_pos;         /* semantic position: j for trunk token j, a_b+i for y_{b,i} */
  int32_t *row_depth;       /* 0 for trunk rows, i for y_{b,i} */
  int32_t *row_trunk_hi;    /* last visible trunk row (packed index): itself, or tree_off+a_b */
  int32_t *row_branch_lo;   /* first visible own-branch row; r+1 (empty) for trunk rows */
  /* per branch [B] (caller order) */
  int32_t *branch_tree;
  int32_t *branch_anchor;   /* local anchor a_b */
  int32_t *branch_len;      /* W_b */
  int32_t *branch_off;      /* packed row of y_{b,1} (for W_b == 1: the next packed row) */
  int32_t *step_off;        /* [B+1] exclusive prefix sum of W_b */
  int32_t *branch_order;    /* [B] branch indices in packed order */
  /* per supervised step [R] */
  int32_t *step_branch;     /* branch of the step */
  int32_t *step_pred_row;   /* packed row whose output predicts the step's sample */
  int32_t *step_sample_row; /* packed row of the sample y_{b,i}; -1 for the terminal sample */
  /* library-internal attention schedule: n_attn_items query blocks of 8 int32,
     then the same blocks in groups of four, (n_attn_items + 3) / 4 + 2 * n_trees
     groups of 4 * 8 int32 */
  int32_t *attn_items;
} spec_tree_layout;

/*
 * spec_tree_pack -- build the packed proposal tree.
 *
 * Defines: [SpecOPD paper page, Figure 2] (a shared reference trunk with
 * sampled continuations attached at their anchors), [SpecOPD paper page,
 * Figure 3] (one packed order; each row sees itself and its ancestors;
 * terminal samples need no query row) and [SpecOPD notes page, "Equations"]
 * (histories h_{b,i} = (x_{<=a_b}, y_{b,<i}); the anchor row predicts y_{b,1},
 * the row of y_{b,i-1} predicts y_{b,i}; semantic position a_b + i).
 *
 * Arguments (all host arrays are read before the call returns):
 *   n_trees       >= 1 trees packed back to back.
 *   h_trunk_len   [n_trees] trunk length T_t >= 1.
 *   h_n_branches  [n_trees] branches per tree (>= 0); B = their sum.
 *   h_anchor      [B] local zero-based anchor, 0 <= a_b < T_t, tree t's
 *                 branches consecutive, trees in order.
 *   h_branch_len  [B] branch width 1 <= W_b <= SPEC_MAX_BRANCH_LEN.
 *   d_mem         device buffer of *mem_bytes bytes for the layout arrays, or
 *                 NULL for a size query (then only the scalars and *mem_bytes
 *                 are written).
 *   mem_bytes     in: size of d_mem; out: bytes required.
 *   layout        out: scalars always; device pointers when d_mem != NULL.
 * Errors: SPEC_ERR_INVALID_ARG for NULL required pointers or out-of-range
 * values (N and R must fit in int32), SPEC_ERR_WORKSPACE when *mem_bytes is
 * too small, SPEC_ERR_HIP when the copy or the expand kernel fails to enqueue.
 */
spec_status spec_tree_pack(int32_t n_trees, const int32_t *h_trunk_len,
                           const int32_t *h_n_branches, const int32_t *h_anchor,
                           const int32_t *h_branch_len, void *d_mem, size_t *mem_bytes,
                           spec_tree_layout *layout, spec_stream stream);

/*
 * spec_tree_attn_fwd -- tree-masked GQA attention over a packed tree.
 *
 * Defines: [SpecOPD paper page, Figure 3] (packed queries share the trunk K/V
 * under a tree mask restricting each row to itself and its ancestors) and
 * [SpecOPD notes page, "Equations"] (only the reference prefix through the
 * anchor and the branch's own predecessors are visible; RoPE uses the
 * semantic position a_b + i, not the packed offset; the readout for step
 * (b,i) is the output row of its predecessor, never the sample's own row).
 *
 * For packed row r and query head h (KV head g = h / (Hq/Hkv)):
 *   O[r,h] = sum_{c in vis(r)} softmax_c(scale * <rope(q[r,h], pos r), rope(k[c,g], pos c)>) v[c,g]
 *   vis(r) = [tree_off[t], row_trunk_hi[r]]  U  [row_branch_lo[r], r]
 * RoPE is rotate-half: dimension j pairs with j + D/2 at angle
 * pos * rope_base^(-2j/D). Accumulation is float32; O is rounded to the input
 * dtype (round-to-nearest-even for bf16).
 *
 * Arguments:
 *   layout        from spec_tree_pack (device arrays must be resident).
 *   n_heads_q     Hq >= 1; n_heads_kv: Hkv >= 1 with Hq % Hkv == 0.
 *   head_dim      D in {32, 64, 128}.
 *   dtype         SPEC_BF16 (MFMA path) or SPEC_F32 (exact float32 path).
 *   d_q           [N, Hq, D]; d_k, d_v: [N, Hkv, D], pre-RoPE, dtype `dtype`.
 *   rope_base     > 0 (e.g. 10000).
 *   softmax_scale <= 0 selects 1/sqrt(D).
 *   d_out         [N, Hq, D] dtype, written for every packed row.
 *   d_readout     optional [R, Hq, D] dtype: readout[s] = O[step_pred_row[s]].
 *   d_work        workspace of *work_bytes bytes, or NULL for a size query.
 * Data precondition (not checked): Q, K, V are finite.
 * Errors: SPEC_ERR_INVALID_ARG, SPEC_ERR_UNSUPPORTED (head_dim / dtype / GQA
 * ratio outside the kernels; bf16 K / V past 4 GiB: all heads for head dims 32
 * and 64, one KV head's rows rounded up to 64 for head dim 128),
 * SPEC_ERR_WORKSPACE, SPEC_ERR_HIP.
 */
spec_status spec_tree_attn_fwd(const spec_tree_layout *layout, int32_t n_heads_q,
                               int32_t n_heads_kv, int32_t head_dim, spec_dtype dtype,
                               const void *d_q, const void *d_k, const void *d_v,
                               float rope_base, float softmax_scale, void *d_out,
                               void *d_readout, void *d_work, size_t *work_bytes,
                               spec_stream stream);

/*
 * spec_qsa_attn_fwd -- sparse attention with branch-consistent indexer groups.
 *
 * Defines: [SpecOPD paper page, Figure 4] (branch-parallel scoring with sparse
 * attention): keys are grouped group_size tokens at a time and each complete
 * group carries an indexer group key; rows reuse the complete groups of the
 * shared trunk; a group holding tokens of the row's own branch is keyed from
 * that branch's history (a branch-specific key, rebuilt per branch); the row's
 * incomplete group is its causal tail; the row's indexer query picks complete
 * groups by top-k and attention reads the picked groups' keys plus the tail,
 * which bypasses top-k.
 *
 * For packed row r at semantic position t (history: trunk positions through the
 * anchor, then the branch's own tokens) and KV head g:
 *   complete groups j < n_c = floor((t + 1) / G); tail = positions n_c*G .. t;
 *   key_j  = mean over the group's positions p of ki[row(p), g];
 *   score_j = <qi[r, g], key_j>; picked = the top_k best (ties: lower j; all if
 *   n_c <= top_k);
 *   O[r, h] for the query heads h of g = softmax attention (as spec_tree_attn_fwd:
 *   rotate-half RoPE at semantic positions, scale) over the keys of the picked
 *   groups and of the tail.
 * Readings the pages leave open: the mean as the group key, one indexer query
 * and key per token and KV head (the pick is shared by the KV head's query
 * heads), the group a row completes counted as complete.
 *
 * Arguments:
 *   layout        from spec_tree_pack (device arrays resident).
 *   n_heads_q, n_heads_kv  Hq % Hkv == 0, Hq / Hkv <= 16.
 *   head_dim      128 (bf16 inputs).
 *   index_dim     DI, a multiple of 8 in [8, 256].
 *   group_size    G >= 1; at most 1024 complete groups per row ((max_pos+1)/G).
 *   top_k         1..64.
 *   d_q [N,Hq,128], d_k / d_v [N,Hkv,128] bf16, pre-RoPE; d_qi / d_ki [N,Hkv,DI]
 *                 bf16 indexer queries and keys (used as given).
 *   rope_base, softmax_scale  as spec_tree_attn_fwd.
 *   d_out         [N,Hq,128] bf16.
 *   d_selected    optional [N,Hkv,top_k] int32 out: the picked groups in
 *                 ascending order, -1 padded (NULL: kept in the workspace).
 *   d_readout     optional [R,Hq,128]: readout[s] = O[step_pred_row[s]].
 *   d_work        workspace of *work_bytes bytes, or NULL for a size query.
 * Scores are summed in float32 in index order; where two groups' float32 scores
 * tie, the lower index wins.
 * Errors: SPEC_ERR_INVALID_ARG, SPEC_ERR_UNSUPPORTED (head_dim, group of query
 * heads, index_dim, group count, sizes past 32-bit offsets), SPEC_ERR_WORKSPACE,
 * SPEC_ERR_HIP.
 */
spec_status spec_qsa_attn_fwd(const spec_tree_layout *layout, int32_t n_heads_q, int32_t n_heads_kv,
                              int32_t head_dim, int32_t index_dim, int32_t group_size, int32_t top_k,
                              const void *d_q, const void *d_k, const void *d_v, const void *d_qi,
                              const void *d_ki, float rope_base, float softmax_scale, void *d_out,
                              int32_t *d_selected, void *d_readout, void *d_work, size_t *work_bytes,
                              spec_stream stream);

/*
 * spec_e2etv_fwd_bwd -- E2E-TV surrogate, loss and gradient w.r.t. the draft.
 *
 * Defines: [SpecOPD notes page, "Equations"]
 *   alpha_s = sum_v min(q_s(v), p_s(v))          (full vocabulary)
 *   L = 1 - inv_norm * sum_b sum_{j=1..W_b} prod_{i<=j} alpha_{b,i}
 * with q = softmax(draft row), p = softmax(teacher row); samples and teacher
 * are held fixed when differentiating, and teacher mass outside the draft
 * support is kept, never renormalised. [SpecOPD notes page, "Inputs and code
 * mapping"]: logits are aligned by history (row s = step s of the layout),
 * low precision is promoted to float32, inactive draft support may be NaN,
 * the teacher must be finite.
 *
 * Gradient written (float32): grad[s,u] = c_s * q_s(u) * (1[q_s(u) < p_s(u)] - S_s)
 * with S_s = sum_{v: q_s(v) < p_s(v)} q_s(v) and c_s = dL/d alpha_s =
 * -inv_norm * A_{b,i-1} * G_{b,i} (prefix products A, suffix sums G).
 *
 * Arguments:
 *   layout        from spec_tree_pack (uses n_steps, n_branches, max_branch_len,
 *                 step_off, step_branch).
 *   vocab         V >= 1.
 *   logit_dtype   SPEC_BF16 or SPEC_F32.
 *   d_draft       [R, V] draft logits z; NaN or -inf mean inactive support (q = 0).
 *   d_teacher     [R, V] teacher logits y, all finite.
 *   inv_norm      <= 0 selects 1/R; otherwise used as given (e.g. a
 *                 normaliser computed across ranks).
 *   d_alpha       [R] float32 out.
 *   d_loss        [1] float32 out.
 *   d_grad        optional [R, V] float32 out (NULL: forward only).
 *   d_work        workspace of *work_bytes bytes, or NULL for a size query.
 * Data preconditions (not checked; violations give NaN): teacher finite, at
 * least one active draft entry per row.
 * For bf16 logits the work runs as one cooperative kernel (8 bytes of memory
 * traffic per logit element) when V is a multiple of 8 and at most 245,760 (a
 * team of at most 16 workgroups splits each row, 15,360 entries apiece), the
 * longest branch is at most one step longer than the number of teams resident
 * on the device (25 on MI355X for V = 151,936) and no team holds more than
 * 2,048 rows. Otherwise,
 * and for float32 logits, three kernels give the same results at about 10
 * bytes per element. The cooperative kernel's workgroups wait on each other
 * through bounded polls; if a poll ever times out (it cannot while the kernel
 * is resident on the device as a whole) alpha and the loss come back NaN and
 * spec_e2etv_status reports it.
 * Calls that share a workspace must not overlap in time.
 * Errors: SPEC_ERR_INVALID_ARG, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP.
 */
spec_status spec_e2etv_fwd_bwd(const spec_tree_layout *layout, int64_t vocab,
                               spec_dtype logit_dtype, const void *d_draft,
                               const void *d_teacher, float inv_norm, float *d_alpha,
                               float *d_loss, float *d_grad, void *d_work, size_t *work_bytes,
                               spec_stream stream);

/*
 * spec_e2etv_status -- the status word of the last E2E-TV call on a workspace.
 *
 * Waits for `stream` (the stream of that call) and copies the call's status
 * word to *h_status: 0 when every bounded wait of its team kernels was met,
 * nonzero when one timed out (alpha and the loss of that call are then NaN).
 * layout and vocab must be those of the call; d_work its workspace, or NULL
 * for the array of spec_e2etv_fwd_bwd_noalloc on the current device.
 * Errors: SPEC_ERR_INVALID_ARG, SPEC_ERR_HIP.
 */
spec_status spec_e2etv_status(const spec_tree_layout *layout, int64_t vocab, const void *d_work,
                              uint32_t *h_status, spec_stream stream);

/*
 * spec_e2etv_fwd_bwd_noalloc -- spec_e2etv_fwd_bwd without a caller workspace.
 *
 * For callers that cannot allocate device memory or hand over a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, results and kernels as spec_e2etv_fwd_bwd (minus
 * d_work / work_bytes); the workspace is a library-owned device array of
 * SPEC_NOALLOC_SCRATCH_BYTES per GPU, held from the library's first use on
 * that GPU until the process ends. The call itself allocates nothing and
 * calls no allocating routine. The kernels clear what must start at zero, so
 * the array may hold anything from an earlier call.
 *
 * Limit: the E2E-TV workspace of (R steps, vocabulary V) must fit the array:
 * 4*4R + 16*8R*2 + 8R bytes plus 256 (about 280 B per step: R up to ~119k) on
 * the fused path (bf16 logits, V a multiple of 8, branches of at most 64
 * steps), plus R * ceil(V/8) bitmask bytes on every other path. Larger
 * requests return SPEC_ERR_UNSUPPORTED with nothing launched.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialised by the
 * caller.
 * Errors: as spec_e2etv_fwd_bwd, plus SPEC_ERR_UNSUPPORTED for the limit
 * above and SPEC_ERR_HIP if the array's device address cannot be looked up.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

spec_status spec_e2etv_fwd_bwd_noalloc(const spec_tree_layout *layout, int64_t vocab,
                                       spec_dtype logit_dtype, const void *d_draft,
                                       const void *d_teacher, float inv_norm, float *d_alpha,
                                       float *d_loss, float *d_grad, spec_stream stream);

/*
 * spec_e2etv_head_fwd_bwd -- E2E-TV with the teacher logits read through an
 * output head: the predecessor readout, the head product and E2E-TV fused, so
 * the teacher logits never reach memory.
 *
 * Defines: [SpecOPD notes page, "Inputs and code mapping"] (prediction logits
 * are formed from hidden states and a head the caller supplies; E2E-TV takes
 * logits aligned by history) and [SpecOPD paper page, Figure 3] (step (b,i)
 * is read from its predecessor's row, the anchor row for i = 1):
 *   y[s, v] = sum_k hidden[step_pred_row[s], k] * head[v, k]
 * then alpha, L and the gradient exactly as spec_e2etv_fwd_bwd with teacher
 * logits y. The products run on bf16 MFMA with float32 sums.
 *
 * Arguments:
 *   layout        from spec_tree_pack (uses n_steps, n_branches,
 *                 max_branch_len, step_off, step_pred_row).
 *   vocab         V >= 8, a multiple of 8.
 *   d_model       hidden size, a positive multiple of 64, at most 2^22; the
 *                 hidden states (N x d_model bf16) must stay under 2 GiB.
 *   draft_dtype   SPEC_BF16 or SPEC_F32: the dtype of d_draft.
 *   d_draft       [R, V] draft logits; NaN or -inf mean inactive support.
 *   d_hidden      [N, d_model] bf16 final hidden states of every packed row
 *                 (N = layout n_rows); only steps' predecessor rows are read.
 *   d_head        [V, d_model] bf16 output head (row v gives logit v).
 *   inv_norm      <= 0 selects 1/R; otherwise used as given.
 *   d_alpha       [R] float32 out; d_loss: [1] float32 out.
 *   d_grad        optional [R, V] float32 out, dL/d draft logits (NULL: forward only).
 *   d_work        workspace of *work_bytes bytes, or NULL for a size query.
 * All device buffers 16-byte aligned. Calls that share a workspace must not
 * overlap in time. Data preconditions (not checked; violations give NaN):
 * hidden and head finite, at least one active draft entry per row.
 * Errors: SPEC_ERR_INVALID_ARG, SPEC_ERR_UNSUPPORTED (vocab or d_model not a
 * multiple of 8 or 64, hidden states of 2 GiB or more, branches longer than 64
 * steps, draft dtype), SPEC_ERR_WORKSPACE, SPEC_ERR_HIP.
 */
spec_status spec_e2etv_head_fwd_bwd(const spec_tree_layout *layout, int64_t vocab,
                                    int32_t d_model, spec_dtype draft_dtype, const void *d_draft,
                                    const void *d_hidden, const void *d_head, float inv_norm,
                                    float *d_alpha, float *d_loss, float *d_grad, void *d_work,
                                    size_t *work_bytes, spec_stream stream);

/*
 * spec_gdn_replay_fwd -- indexed GDN state replay: the linear-attention
 * (GDN) outputs of every branch row.
 *
 * Defines: [SpecOPD paper page, Figure 5] (GDN scoring of branches from stored
 * trunk states): the trunk runs once and its FP32 state is stored every `chunk`
 * tokens; a branch takes the last stored state at or before its anchor, runs
 * the remaining trunk tokens up to the anchor on its own copy, then runs its
 * own tokens, producing one output per token; the replay never writes a stored
 * state, and each token's convolution window runs over its ancestors.
 * [SpecOPD paper page, Figure 13]: the replayed trunk tokens count as GDN work.
 *
 * The pages do not write the recurrence out; this is the gated delta rule,
 * per head, with state S (D x D, value rows i, key columns j):
 *   S_ij <- alpha S_ij + beta (v_i - alpha sum_j' S_ij' k_j') k_j,
 *   o_i   = sum_j S_ij q_j   (after the update),
 * on features that are, per token and head, a depthwise convolution of width
 * K along the ancestry path (tap m on the m-th ancestor: the token itself,
 * its parent, ...; nothing before the tree's first token), then SiLU, with q
 * and k then L2-normalised over D and q scaled by 1/sqrt(D).
 * Checkpoint c of tree t is S after trunk tokens 0 .. c*chunk-1 (c = 0: the
 * zero state); a branch anchored at a starts from c = (a + 1) / chunk.
 *
 * Arguments:
 *   layout      from spec_tree_pack (uses n_trees, n_branches, max_trunk_len,
 *               tree_off, branch_tree, branch_anchor, branch_len, branch_off;
 *               the trunk pass also tree_trunk_len).
 *   n_heads     H >= 1; head_dim D in {64, 128}; conv_width K in 1..4;
 *               chunk >= 1 (the checkpoint spacing C).
 *   d_xq, d_xk, d_xv  [N, H, D] bf16: q, k, v projections of every packed
 *               row before the convolution.
 *   d_taps      [3, H, D, K] float32: taps of the q, k and v convolutions.
 *   d_alpha     [N, H] float32, the decay alpha in (0, 1]; d_beta [N, H]
 *               float32, the write strength.
 *   d_ckpt      [n_trees, max_trunk_len / chunk + 1, H, D, D] float32, each
 *               state stored key-major (S_ij at j * D + i); slots a shorter
 *               tree never reaches are not read.
 *   d_trunk_work  NULL, or the workspace of the spec_gdn_trunk_fwd call (same
 *               layout, H, D, K and chunk <= 64) that wrote d_ckpt, unchanged
 *               since. With it the replay runs a chunk at a time: the trunk
 *               pass's per-token deltas of the anchor's chunk stand in for the
 *               replayed trunk tokens (S after the anchor = e^G S_c + sum of
 *               their decayed rank-one updates), and the branch's tokens form
 *               one more chunk (same result up to float32 rounding). Without it
 *               one workgroup per (branch, head, row block) walks the tokens one
 *               at a time.
 *   d_out       [N, H, D] float32: the rows of branches are written; trunk
 *               rows are left as they are (the trunk pass owns them).
 * All buffers are the caller's; the call allocates nothing. Data
 * preconditions (not checked): inputs finite; the convolved q and k of every
 * replayed token are not all zero (their norms divide).
 * Errors: SPEC_ERR_INVALID_ARG (also a trunk cache with chunk > 64),
 * SPEC_ERR_UNSUPPORTED (head_dim, conv_width), SPEC_ERR_HIP.
 */
spec_status spec_gdn_replay_fwd(const spec_tree_layout *layout, int32_t n_heads,
                                int32_t head_dim, int32_t conv_width, int32_t chunk,
                                const void *d_xq, const void *d_xk, const void *d_xv,
                                const float *d_taps, const float *d_alpha, const float *d_beta,
                                const float *d_ckpt, const void *d_trunk_work, float *d_out,
                                spec_stream stream);

/*
 * spec_gdn_trunk_fwd -- the shared trunk pass of GDN scoring: the GDN outputs
 * of every trunk row and the checkpoints spec_gdn_replay_fwd reads.
 *
 * Defines: [SpecOPD paper page, Figure 5] (the one pass over the trunk that
 * stores the FP32 GDN state every `chunk` tokens). Same recurrence, features and
 * argument meanings as spec_gdn_replay_fwd, along each tree's trunk from the
 * zero state: o is written for every trunk row, and slot c of d_ckpt (key-major
 * state, layout as for spec_gdn_replay_fwd) receives the state after trunk
 * tokens 0 .. c*chunk-1 for c = 0 .. T_t / chunk. Slots a shorter tree never
 * reaches are left as they are. Branch rows of d_out are left as they are.
 *
 * For chunk <= 64 the pass runs a chunk at a time: the chunks' S0-independent
 * parts (features, the in-chunk triangular system, the output and state
 * coefficients) in parallel, then one ordered pass over the chunks per head
 * that carries the state, then the outputs in parallel; the result equals the
 * token-at-a-time recurrence up to float32 rounding. For chunk > 64 one
 * workgroup per (tree, head, row block) walks the trunk a token at a time.
 *
 * Arguments: as spec_gdn_replay_fwd, plus
 *   d_ckpt      [n_trees, max_trunk_len / chunk + 1, H, D, D] float32, written.
 *   d_out       [N, H, D] float32; trunk rows written.
 *   d_work      workspace of *work_bytes bytes (16-byte aligned), or NULL for a
 *               size query (then nothing else is read). The chunked pass keeps
 *               seven 64 x D float32 tiles and 65 floats per (tree, chunk, head)
 *               there; spec_gdn_replay_fwd can read them (d_trunk_work).
 * Calls that share a workspace must not overlap in time.
 * Errors: as spec_gdn_replay_fwd, plus SPEC_ERR_WORKSPACE.
 */
spec_status spec_gdn_trunk_fwd(const spec_tree_layout *layout, int32_t n_heads, int32_t head_dim,
                               int32_t conv_width, int32_t chunk, const void *d_xq,
                               const void *d_xk, const void *d_xv, const float *d_taps,
                               const float *d_alpha, const float *d_beta, float *d_ckpt,
                               float *d_out, void *d_work, size_t *work_bytes,
                               spec_stream stream);

/*
 * Measurement hook (benchmarks only; it changes no result).
 *
 * After spec_profile_attach(p) on a thread, every call on that thread records
 * p->events[p->used] on the call's stream once before its first kernel (name
 * "<call>:begin") and once after each kernel it launches (name = the kernel),
 * incrementing p->used, until p->capacity events are used. The time between
 * consecutive events is then one kernel's duration. Events are hipEvent_t
 * handles created by the caller; names are static strings. Pass NULL to detach.
 */
#define SPEC_PROFILE_MAX 256
typedef struct spec_profile {
  void **events;                        /* [capacity] hipEvent_t, caller-created */
  int32_t capacity;                     /* <= SPEC_PROFILE_MAX */
  int32_t used;                         /* out: events recorded so far */
  const char *names[SPEC_PROFILE_MAX];  /* out: what ended at events[i] */
} spec_profile;

void spec_profile_attach(spec_profile *p);

/* Human-readable name of a status code (static string). */
const char *spec_status_string(spec_status status);

/* Description of the last error raised on the calling thread ("" if none). */
const char *spec_last_error(void);

/* SPEC_TREE_ABI_VERSION of the loaded library. */
int32_t spec_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_TREE_H */
