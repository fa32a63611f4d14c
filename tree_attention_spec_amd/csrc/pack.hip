// Proposal-tree pack: host checks and O(B) prefix sums, device expansion of
// the per-row and per-step arrays.
//
// [SpecOPD paper page, Figure 2]: branches hang off anchors on a shared trunk.
// [SpecOPD paper page, Figure 3]: one packed order for rows and columns; each
// row sees itself and its ancestors; terminal samples have no query row.
// [SpecOPD notes page, "Equations"]: the anchor row predicts y_{b,1}, the row
// of y_{b,i-1} predicts y_{b,i}; y_{b,i} sits at semantic position a_b + i.
#include <algorithm>
#include <array>
#include <cstring>
#include <cstdarg>
#include <cstdio>
#include <numeric>
#include <vector>

#include "common.h"

namespace spec {

// ---------------------------------------------------------------- expand kernels

// One thread per trunk row: grid.y = tree, x covers j in [0, T_t).
__global__ void pack_expand_trunk(const int32_t *__restrict__ tree_off,
                                  const int32_t *__restrict__ tree_len, int32_t *row_tree,
                                  int32_t *row_branch, int32_t *row_anchor, int32_t *row_pos,
                                  int32_t *row_depth, int32_t *row_trunk_hi,
                                  int32_t *row_branch_lo) {
  const int t = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= tree_len[t]) return;
  const int r = tree_off[t] + j;
  row_tree[r] = t;
  row_branch[r] = -1;
  row_anchor[r] = -1;
  row_pos[r] = j;
  row_depth[r] = 0;
  row_trunk_hi[r] = r;        // a trunk row sees the trunk through itself
  row_branch_lo[r] = r + 1;   // and no branch rows
}

// One thread per (branch, i), i in [0, max_branch_len): step i+1 of branch b
// and, for i < W_b - 1, the packed row of y_{b,i+1}.
__global__ void pack_expand_branches(int32_t n_branches, int32_t max_len,
                                     const int32_t *__restrict__ tree_off,
                                     const int32_t *__restrict__ branch_tree,
                                     const int32_t *__restrict__ branch_anchor,
                                     const int32_t *__restrict__ branch_len,
                                     const int32_t *__restrict__ branch_off,
                                     const int32_t *__restrict__ step_off, int32_t *row_tree,
                                     int32_t *row_branch, int32_t *row_anchor, int32_t *row_pos,
                                     int32_t *row_depth, int32_t *row_trunk_hi,
                                     int32_t *row_branch_lo, int32_t *step_branch,
                                     int32_t *step_pred_row, int32_t *step_sample_row) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int b = (int)(idx / max_len);
  const int i = (int)(idx % max_len);  // zero-based: this thread owns sample y_{b,i+1}
  if (b >= n_branches) return;
  const int w = branch_len[b];
  if (i >= w) return;
  const int t = branch_tree[b];
  const int a = branch_anchor[b];
  const int off = branch_off[b];
  const int s = step_off[b] + i;
  step_branch[s] = b;
  step_pred_row[s] = (i == 0) ? tree_off[t] + a : off + i - 1;
  step_sample_row[s] = (i < w - 1) ? off + i : -1;
  if (i < w - 1) {
    const int r = off + i;
    row_tree[r] = t;
    row_branch[r] = b;
    row_anchor[r] = a;
    row_pos[r] = a + i + 1;
    row_depth[r] = i + 1;
    row_trunk_hi[r] = tree_off[t] + a;  // the trunk through the anchor
    row_branch_lo[r] = off;             // and its own branch from y_{b,1}
  }
}

hipError_t launch_pack_expand(const spec_tree_layout &L, const int32_t *d_tree_len,
                              int32_t max_trunk, hipStream_t stream) {
  if (max_trunk > 0) {
    dim3 grid((max_trunk + 255) / 256, L.n_trees);
    hipLaunchKernelGGL(pack_expand_trunk, grid, dim3(256), 0, stream, L.tree_off, d_tree_len,
                       L.row_tree, L.row_branch, L.row_anchor, L.row_pos, L.row_depth,
                       L.row_trunk_hi, L.row_branch_lo);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (L.n_branches > 0) {
    const int64_t n = (int64_t)L.n_branches * L.max_branch_len;
    hipLaunchKernelGGL(pack_expand_branches, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, L.n_branches, L.max_branch_len, L.tree_off, L.branch_tree,
                       L.branch_anchor, L.branch_len, L.branch_off, L.step_off, L.row_tree,
                       L.row_branch, L.row_anchor, L.row_pos, L.row_depth, L.row_trunk_hi,
                       L.row_branch_lo, L.step_branch, L.step_pred_row, L.step_sample_row);
    return hipGetLastError();
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- host planning

namespace {

struct Plan {
  int32_t n_trees = 0, B = 0, max_len = 0, max_pos = -1, max_trunk = 0;
  int64_t N = 0, R = 0;
  // host images of the arrays copied to the device, in carve order
  std::vector<int32_t> tree_off, tree_len, branch_tree, branch_anchor, branch_len, branch_off,
      step_off, branch_order;
  std::vector<AttnItem> items;
  std::vector<AttnItem> groups;  // attn_group_count groups of kAttnGroup blocks
};

// Query blocks for the attention kernel, longest first. Trunk blocks take 32
// consecutive trunk rows; branch blocks take 32 consecutive branch rows of a
// tree (branches are anchor-sorted, so a block's anchors are close together).
void plan_attention(Plan &p) {
  const int BR = kAttnBlockRows;
  // groups of up to kAttnGroup consecutive blocks of one tree's trunk or branch rows
  std::vector<std::pair<int32_t, std::array<AttnItem, kAttnGroup>>> groups;  // (cost, blocks)
  size_t run = 0;  // first block of the current run of one tree's trunk or branch rows
  auto close_run = [&]() {
    for (size_t i = run; i < p.items.size(); i += kAttnGroup) {
      std::array<AttnItem, kAttnGroup> g{};
      int32_t cost = 0;
      for (size_t j = 0; j < (size_t)kAttnGroup && i + j < p.items.size(); ++j) {
        g[j] = p.items[i + j];
        cost = std::max(cost, g[j].cost);
      }
      groups.emplace_back(cost, g);
    }
    run = p.items.size();
  };
  int k = 0;  // position in packed branch order
  for (int t = 0; t < p.n_trees; ++t) {
    const int off = p.tree_off[t], T = p.tree_len[t];
    for (int q0 = off; q0 < off + T; q0 += BR) {
      AttnItem it{};
      it.q0 = q0;
      it.q1 = std::min(q0 + BR, off + T);
      it.tk0 = off;
      it.tk1 = it.q1;
      it.tfull = q0 + 1;  // the first query of the block sees keys <= q0
      it.bk0 = it.bk1 = 0;
      it.cost = it.tk1 - it.tk0;
      p.items.push_back(it);
    }
    close_run();
    // branches of tree t in packed order: branch_order[k .. k_end)
    int k_end = k;
    while (k_end < p.B && p.branch_tree[p.branch_order[k_end]] == t) ++k_end;
    const int bstart = off + T, bend = p.tree_off[t + 1];
    int kf = k;  // first branch whose rows reach past q0
    for (int q0 = bstart; q0 < bend; q0 += BR) {
      const int q1 = std::min(q0 + BR, bend);
      auto row_end = [&](int kk) {
        const int b = p.branch_order[kk];
        return p.branch_off[b] + p.branch_len[b] - 1;
      };
      while (row_end(kf) <= q0) ++kf;  // skips finished and one-token branches
      int kl = kf;
      while (row_end(kl) < q1) ++kl;
      const int bf = p.branch_order[kf], bl = p.branch_order[kl];
      AttnItem it{};
      it.q0 = q0;
      it.q1 = q1;
      it.tk0 = off;
      it.tk1 = off + p.branch_anchor[bl] + 1;   // largest anchor in the block
      it.tfull = off + p.branch_anchor[bf] + 1; // smallest anchor in the block
      it.bk0 = p.branch_off[bf];
      it.bk1 = q1;
      it.cost = (it.tk1 - it.tk0) + (it.bk1 - it.bk0);
      p.items.push_back(it);
    }
    close_run();
    k = k_end;
  }
  std::stable_sort(p.items.begin(), p.items.end(),
                   [](const AttnItem &a, const AttnItem &b) { return a.cost > b.cost; });
  std::stable_sort(groups.begin(), groups.end(),
                   [](const auto &a, const auto &b) { return a.first > b.first; });
  const int64_t n_groups = attn_group_count((int64_t)p.items.size(), p.n_trees);
  p.groups.assign((size_t)n_groups * kAttnGroup, AttnItem{});
  for (size_t i = 0; i < groups.size(); ++i)
    for (int j = 0; j < kAttnGroup; ++j) p.groups[i * kAttnGroup + j] = groups[i].second[j];
}

spec_status make_plan(int32_t n_trees, const int32_t *h_trunk_len, const int32_t *h_n_branches,
                      const int32_t *h_anchor, const int32_t *h_branch_len, Plan &p) {
  if (n_trees < 1) return fail(SPEC_ERR_INVALID_ARG, "n_trees must be >= 1 (got %d)", n_trees);
  if (!h_trunk_len || !h_n_branches)
    return fail(SPEC_ERR_INVALID_ARG, "h_trunk_len and h_n_branches must be non-NULL");
  p.n_trees = n_trees;
  int64_t B = 0;
  for (int t = 0; t < n_trees; ++t) {
    if (h_trunk_len[t] < 1)
      return fail(SPEC_ERR_INVALID_ARG, "tree %d: trunk length %d < 1", t, h_trunk_len[t]);
    if (h_n_branches[t] < 0)
      return fail(SPEC_ERR_INVALID_ARG, "tree %d: negative branch count", t);
    B += h_n_branches[t];
  }
  if (B > INT32_MAX / 2) return fail(SPEC_ERR_INVALID_ARG, "too many branches");
  if (B > 0 && (!h_anchor || !h_branch_len))
    return fail(SPEC_ERR_INVALID_ARG, "h_anchor and h_branch_len must be non-NULL when B > 0");
  p.B = (int32_t)B;
  p.tree_off.resize(n_trees + 1);
  p.tree_len.assign(h_trunk_len, h_trunk_len + n_trees);
  p.branch_tree.resize(B);
  p.branch_anchor.assign(h_anchor, h_anchor + B);
  p.branch_len.assign(h_branch_len, h_branch_len + B);
  p.branch_off.resize(B);
  p.step_off.resize(B + 1);
  p.branch_order.resize(B);

  int64_t b = 0, rows = 0;
  for (int t = 0; t < n_trees; ++t) {
    const int T = h_trunk_len[t];
    p.max_trunk = std::max(p.max_trunk, T);
    p.max_pos = std::max(p.max_pos, T - 1);
    for (int64_t e = b + h_n_branches[t]; b < e; ++b) {
      const int a = h_anchor[b], w = h_branch_len[b];
      if (a < 0 || a >= T)
        return fail(SPEC_ERR_INVALID_ARG, "branch %lld: anchor %d outside [0, %d)", (long long)b, a, T);
      if (w < 1 || w > SPEC_MAX_BRANCH_LEN)
        return fail(SPEC_ERR_INVALID_ARG, "branch %lld: width %d outside [1, %d]", (long long)b, w,
                    SPEC_MAX_BRANCH_LEN);
      p.branch_tree[b] = t;
      p.max_len = std::max(p.max_len, w);
      p.max_pos = std::max(p.max_pos, a + w - 1);
      rows += w - 1;
    }
    rows += T;
  }
  p.N = rows;
  p.R = 0;
  for (int64_t i = 0; i < B; ++i) p.R += h_branch_len[i];
  if (p.N > INT32_MAX - 64 || p.R > INT32_MAX - 64)
    return fail(SPEC_ERR_INVALID_ARG, "N=%lld or R=%lld does not fit in int32", (long long)p.N,
                (long long)p.R);

  // packed order: per tree the trunk, then its branches by ascending anchor (stable)
  int32_t cur = 0;
  int64_t first = 0;
  for (int t = 0; t < n_trees; ++t) {
    p.tree_off[t] = cur;
    cur += h_trunk_len[t];
    const int64_t nb = h_n_branches[t];
    int32_t *ord = p.branch_order.data() + first;
    std::iota(ord, ord + nb, (int32_t)first);
    std::stable_sort(ord, ord + nb, [&](int32_t x, int32_t y) { return h_anchor[x] < h_anchor[y]; });
    for (int64_t k = 0; k < nb; ++k) {
      p.branch_off[ord[k]] = cur;
      cur += h_branch_len[ord[k]] - 1;
    }
    first += nb;
  }
  p.tree_off[n_trees] = cur;
  p.step_off[0] = 0;
  for (int64_t i = 0; i < B; ++i) p.step_off[i + 1] = p.step_off[i] + h_branch_len[i];
  plan_attention(p);
  return SPEC_OK;
}

// Carve order of d_mem. The first group is copied from the host, the second
// is written by the expand kernels.
struct Carve {
  size_t off_tree_off, off_tree_len, off_branch_tree, off_branch_anchor, off_branch_len,
      off_branch_off, off_step_off, off_branch_order, off_items, head_bytes;
  size_t off_rows[7];
  size_t off_steps[3];
  size_t total;
};

Carve carve(const Plan &p) {
  Carve c{};
  size_t o = 0;
  auto take = [&](size_t n_ints) {
    size_t at = o;
    o = align_up(o + n_ints * sizeof(int32_t), 256);
    return at;
  };
  c.off_tree_off = take(p.n_trees + 1);
  c.off_tree_len = take(p.n_trees);
  c.off_branch_tree = take(p.B);
  c.off_branch_anchor = take(p.B);
  c.off_branch_len = take(p.B);
  c.off_branch_off = take(p.B);
  c.off_step_off = take(p.B + 1);
  c.off_branch_order = take(p.B);
  c.off_items = take((p.items.size() + p.groups.size()) * kAttnItemInts);
  c.head_bytes = o;
  for (auto &r : c.off_rows) r = take(p.N);
  for (auto &s : c.off_steps) s = take(p.R);
  c.total = o;
  return c;
}

}  // namespace

}  // namespace spec

using namespace spec;

extern "C" spec_status spec_tree_pack(int32_t n_trees, const int32_t *h_trunk_len,
                                      const int32_t *h_n_branches, const int32_t *h_anchor,
                                      const int32_t *h_branch_len, void *d_mem,
                                      size_t *mem_bytes, spec_tree_layout *layout,
                                      spec_stream stream) {
  clear_error();
  if (!layout || !mem_bytes) return fail(SPEC_ERR_INVALID_ARG, "layout and mem_bytes must be non-NULL");
  Plan p;
  spec_status st = make_plan(n_trees, h_trunk_len, h_n_branches, h_anchor, h_branch_len, p);
  if (st != SPEC_OK) return st;
  const Carve c = carve(p);

  spec_tree_layout L{};
  L.n_trees = p.n_trees;
  L.n_branches = p.B;
  L.max_branch_len = p.max_len;
  L.max_pos = p.max_pos;
  L.n_rows = p.N;
  L.n_steps = p.R;
  L.n_attn_items = (int32_t)p.items.size();
  L.max_trunk_len = p.max_trunk;
  if (!d_mem) {  // size query: scalars only, no HIP call
    *mem_bytes = c.total;
    *layout = L;
    return SPEC_OK;
  }
  if (*mem_bytes < c.total) {
    size_t have = *mem_bytes;
    *mem_bytes = c.total;
    return fail(SPEC_ERR_WORKSPACE, "layout buffer has %zu bytes, needs %zu", have, c.total);
  }
  if (!aligned16(d_mem)) return fail(SPEC_ERR_INVALID_ARG, "d_mem must be 16-byte aligned");

  char *base = static_cast<char *>(d_mem);
  auto at = [&](size_t off) { return reinterpret_cast<int32_t *>(base + off); };
  L.tree_off = at(c.off_tree_off);
  L.tree_trunk_len = at(c.off_tree_len);
  L.branch_tree = at(c.off_branch_tree);
  L.branch_anchor = at(c.off_branch_anchor);
  L.branch_len = at(c.off_branch_len);
  L.branch_off = at(c.off_branch_off);
  L.step_off = at(c.off_step_off);
  L.branch_order = at(c.off_branch_order);
  L.attn_items = at(c.off_items);
  int32_t **rows[7] = {&L.row_tree, &L.row_branch, &L.row_anchor, &L.row_pos,
                       &L.row_depth, &L.row_trunk_hi, &L.row_branch_lo};
  for (int i = 0; i < 7; ++i) *rows[i] = at(c.off_rows[i]);
  int32_t **steps[3] = {&L.step_branch, &L.step_pred_row, &L.step_sample_row};
  for (int i = 0; i < 3; ++i) *steps[i] = at(c.off_steps[i]);

  // host image of the head group, one copy
  std::vector<char> head(c.head_bytes, 0);
  auto put = [&](size_t off, const void *src, size_t bytes) {
    if (bytes) std::memcpy(head.data() + off, src, bytes);
  };
  put(c.off_tree_off, p.tree_off.data(), p.tree_off.size() * 4);
  put(c.off_tree_len, p.tree_len.data(), p.tree_len.size() * 4);
  put(c.off_branch_tree, p.branch_tree.data(), p.branch_tree.size() * 4);
  put(c.off_branch_anchor, p.branch_anchor.data(), p.branch_anchor.size() * 4);
  put(c.off_branch_len, p.branch_len.data(), p.branch_len.size() * 4);
  put(c.off_branch_off, p.branch_off.data(), p.branch_off.size() * 4);
  put(c.off_step_off, p.step_off.data(), p.step_off.size() * 4);
  put(c.off_branch_order, p.branch_order.data(), p.branch_order.size() * 4);
  put(c.off_items, p.items.data(), p.items.size() * sizeof(AttnItem));
  put(c.off_items + p.items.size() * sizeof(AttnItem), p.groups.data(), p.groups.size() * sizeof(AttnItem));

  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_mark(s, "pack:begin");
  SPEC_HIP_TRY(hipMemcpyAsync(d_mem, head.data(), c.head_bytes, hipMemcpyHostToDevice, s));
  prof_mark(s, "pack_copy");
  SPEC_HIP_TRY(launch_pack_expand(L, at(c.off_tree_len), p.max_trunk, s));
  prof_mark(s, "pack_expand");
  *mem_bytes = c.total;
  *layout = L;
  return SPEC_OK;
}
