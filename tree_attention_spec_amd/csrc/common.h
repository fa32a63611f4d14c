// Internal helpers shared by the translation units of libspec_tree.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "spec_tree.h"

namespace spec {

// ---------------------------------------------------------------- error reporting
// Record a message for spec_last_error() on the calling thread and return `s`.
spec_status fail(spec_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
spec_status hip_fail(hipError_t e, const char *what);

#define SPEC_HIP_TRY(expr)                                  \
  do {                                                      \
    hipError_t e_ = (expr);                                 \
    if (e_ != hipSuccess) return ::spec::hip_fail(e_, #expr); \
  } while (0)

// Record a profiling event (no-op unless a spec_profile is attached on this thread).
void prof_mark(hipStream_t s, const char *name);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- attention schedule
// One query block of the tree-attention kernel. Query rows [q0, q1) (packed,
// at most kAttnBlockRows) attend to trunk keys [tk0, tk1) and branch keys
// [bk0, bk1). Every query of the block sees every trunk key below `tfull`,
// so tiles that end at or below it need no mask.
struct AttnItem {
  int32_t q0, q1, tk0, tk1, tfull, bk0, bk1, cost;
};
static_assert(sizeof(AttnItem) == 32, "AttnItem is 8 int32");
constexpr int kAttnBlockRows = 32;
constexpr int kAttnItemInts = 8;
// The same blocks grouped kAttnGroup at a time, for the tiled attention with one
// or two query heads per KV head (whose workgroups then take several blocks of one
// KV head and share each K/V tile among them): a group holds consecutive blocks of
// one tree's trunk rows or of one tree's branch rows, in row order, padded with
// empty blocks (q0 == q1 == 0); groups are ordered longest first and padded to
// attn_group_count groups with empty ones. They follow the n_attn_items blocks in
// the layout's attn_items.
constexpr int kAttnGroup = 4;
__host__ __device__ inline int64_t attn_group_count(int64_t n_items, int64_t n_trees) {
  return (n_items + kAttnGroup - 1) / kAttnGroup + 2 * n_trees;
}

// ---------------------------------------------------------------- launchers (per TU)
hipError_t launch_pack_expand(const spec_tree_layout &L, const int32_t *d_tree_len, int32_t max_trunk,
                              hipStream_t stream);

hipError_t launch_rope_table(float2 *tab, int32_t n_pos, int32_t half_dim, double base,
                             hipStream_t stream);
hipError_t launch_rope_k(const void *k, void *kws, const float2 *tab, const int32_t *row_pos,
                         int64_t n_rows, int32_t hkv, int32_t head_dim, spec_dtype dtype,
                         hipStream_t stream);
hipError_t launch_tree_attn(const spec_tree_layout &L, int32_t hq, int32_t hkv, int32_t head_dim,
                            spec_dtype dtype, const void *q, const void *kws, const void *v,
                            const float2 *tab, float scale, void *out, hipStream_t stream);
// Head dim 128, bf16: K rotated and V transposed into 64-key tiles (rope.hip),
// read by the tiled attention kernel (attn.hip).
constexpr int kKeyTile = 64;
// Slot swizzle of the V^T key tiles: chunk c (8 keys) of dim d is stored in
// slot d*8 + (c ^ vt_swizzle(d)). Any 16 consecutive dims reading one chunk
// then fall in 16 distinct 16-byte bank groups of LDS, and so do any 8 (a
// 128-bit LDS read is served 16 lanes at a time).
__device__ __host__ inline int vt_swizzle(int d) { return (d & 7) ^ ((d >> 3) & 1); }
hipError_t launch_kv_tiles(const void *k, const void *v, void *kt, void *vt, const float2 *tab,
                           const int32_t *row_pos, int64_t n_rows, int32_t hkv, hipStream_t stream);
hipError_t launch_tree_attn_tiled(const spec_tree_layout &L, int32_t hq, int32_t hkv, const void *q,
                                  const void *kt, const void *vt, const float2 *tab, float scale,
                                  void *out, hipStream_t stream);
hipError_t launch_readout(const int32_t *pred_row, int64_t n_steps, int64_t row_bytes,
                          const void *out, void *readout, hipStream_t stream);

// Statistics teams: at most kTeamMax members per row.
constexpr int kTeamMax = 16;

struct E2etvWork {
  float *lse_q2;   // [R] log2-domain log-sum-exp of the draft row
  float *lse_p2;   // [R] same for the teacher
  float *S;        // [R] sum of q over {q < p}
  float *coef;     // [R] dL/d alpha
  float2 *part;    // [R][team] (alpha, S) partials of the members of a statistics team
  unsigned long long *xchg;  // [R][team] log-sum-exp slots the members of a team exchange
  unsigned *status;          // [0] raised if a team exchange timed out; [1] the scan kernel's ticket
  double *branch_sum;        // [R] per-branch sum of prefix products (at most R branches)
  uint8_t *bits;   // [R][bits_row] bit u of a row: 1 iff q_u < p_u (the set S is summed over)
  int64_t bits_row;
};
size_t e2etv_work_bytes(int64_t n_steps, int64_t vocab);
// Bytes of the workspace before the {q < p} bitmask: all the fused path uses.
size_t e2etv_work_bytes_fused(int64_t n_steps);
E2etvWork e2etv_carve(void *d_work, int64_t n_steps, int64_t vocab);
// Whether launch_e2etv runs the fused pipeline (which never touches w.bits) for
// this layout, vocabulary and dtype on the current device.
hipError_t e2etv_takes_fused_path(const spec_tree_layout &L, int64_t vocab, spec_dtype dtype, bool *fused);
hipError_t launch_e2etv(const spec_tree_layout &L, int64_t vocab, spec_dtype dtype,
                        const void *draft, const void *teacher, float inv_norm, float *alpha,
                        float *loss, float *grad, const E2etvWork &w, hipStream_t stream);
// The scan (prefix products, dL/d alpha, L) and gradient stages alone, for a
// path with its own statistics kernels: w.part holds [R][team] (alpha, S)
// partials summed in member order, w.lse_q2 the draft log-sum-exps, w.bits the
// {q < p} bitmask, and w.status[1] (the scan's ticket) is zero. vocab % 8 == 0.
hipError_t launch_e2etv_tail(const spec_tree_layout &L, int64_t vocab, spec_dtype dtype,
                             const void *draft, float inv_norm, int team, float *alpha,
                             float *loss, float *grad, const E2etvWork &w, hipStream_t stream);

// Sparse attention with branch-consistent indexer groups (head dim 128, bf16):
// group keys, top-k picks and attention over the picked groups plus the causal
// tail, reading the K / V^T tiles of launch_kv_tiles.
size_t qsa_keys_floats(const spec_tree_layout &L, int32_t hkv, int32_t index_dim, int32_t group_size);
hipError_t launch_qsa(const spec_tree_layout &L, int32_t hq, int32_t hkv, int32_t index_dim,
                      int32_t group_size, int32_t top_k, const void *q, const void *qi, const void *ki,
                      const void *kt, const void *vt, const float2 *tab, float scale, float *keys,
                      int32_t *sel, void *out, hipStream_t stream);

// E2E-TV with the teacher logits formed from hidden states and an output head.
size_t e2etv_head_work_bytes(int64_t n_steps, int64_t vocab);
hipError_t launch_e2etv_head(const spec_tree_layout &L, int64_t vocab, int32_t d_model,
                             spec_dtype draft_dtype, const void *draft, const void *hidden,
                             const void *head, float inv_norm, float *alpha, float *loss,
                             float *grad, void *work, hipStream_t stream);

}  // namespace spec
