// Sparse attention with branch-consistent indexer groups over a packed tree.
//
// [SpecOPD paper page, Figure 4]: keys are grouped G tokens at a time and every
// complete group carries an indexer group key; a row reuses the complete groups
// of the shared trunk, a group that holds tokens of the row's own branch gets a
// key built from that branch's history (rebuilt per branch), the row's
// incomplete group stays in its causal tail, and attention reads the keys of the
// top-k groups its indexer query picks plus the tail, which bypasses top-k.
//
// For a row at semantic position t (trunk token t, or y_{b,i} at t = a_b + i) the
// groups cover positions [jG, (j+1)G) of its history; groups j < floor((t+1)/G)
// are complete (the one the row completes included) and positions
// floor((t+1)/G)*G .. t form the tail. A group key is the mean of the group's
// per-token indexer keys; group j scores <indexer query of the row, key j>; the
// k best scores are picked (ties: lower j). One indexer query and key per token
// and KV head: the pick is shared by that KV head's query heads.
//
// Three kernels after the RoPE table and the K / V^T tile pre-pass of the full
// attention path (rope.hip):
//   qsa_keys_kernel    the group keys: every complete trunk group of each tree
//                      once (stored dim-major, a tree's groups contiguous per
//                      dim), and for each branch the groups that hold its
//                      tokens (at most ceil((W_b - 1)/G)), one wave per key
//   qsa_select_kernel  one wave per (row, KV head), a workgroup per KV head and
//                      4 rows: scores of every complete
//                      group (trunk keys below the branch's first own group,
//                      the branch's keys from there), exact top-k by k rounds of
//                      a wave arg-max, picks written in ascending order
//   qsa_attn_kernel    one wave per (row, KV head): the picked groups and the
//                      tail as packed-row ranges (a group that straddles the
//                      anchor is two ranges), read 32 keys at a time straight
//                      from the tiles into MFMA fragments (no LDS: the rows of
//                      a block share no keys), v_mfma_f32_16x16x32_bf16 with the
//                      KV head's query heads as the 16 columns, online softmax.
#include "common.h"

namespace spec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQsaD = 128;
constexpr int kQsaWaves = 4;          // waves (items) per workgroup
constexpr float kQsaLazyMax = 8.f;    // log2 headroom of the softmax reference

__device__ inline float bf(const __bf16 x) { return (float)x; }

// ---------------------------------------------------------------- group keys
// Item i < n_trunk_items: tree t = i / max_tg, trunk group j = i % max_tg;
// otherwise branch b = (i - n_trunk_items) / max_bg, its s-th own group. A
// lane sums index dims lane, lane + 64, ... over the group's tokens in order.
__global__ __launch_bounds__(64 * kQsaWaves) void qsa_keys_kernel(
    const __bf16 *__restrict__ ki, int32_t hkv, int32_t di, int32_t G, const int32_t *__restrict__ tree_off,
    const int32_t *__restrict__ tree_len, int32_t n_trees, int32_t max_tg, const int32_t *__restrict__ branch_tree,
    const int32_t *__restrict__ branch_anchor, const int32_t *__restrict__ branch_len,
    const int32_t *__restrict__ branch_off, int32_t n_branches, int32_t max_bg, int32_t tg_stride,
    float *__restrict__ trunk_keys, float *__restrict__ branch_keys) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kQsaWaves + (threadIdx.x >> 6);
  const int64_t n_trunk_items = (int64_t)n_trees * max_tg;
  const int64_t n_items = n_trunk_items + (int64_t)n_branches * max_bg;
  if (item >= n_items * hkv) return;
  const int g = (int)(item % hkv);
  const int64_t slot = item / hkv;
  int base, anchor, boff, j;
  float *dst;
  int64_t dstride;  // floats between consecutive dims of this key
  if (slot < n_trunk_items) {
    const int t = (int)(slot / max_tg);
    j = (int)(slot % max_tg);
    if ((j + 1) * G > tree_len[t]) return;  // not a complete group of this tree
    base = tree_off[t];
    anchor = INT32_MAX;
    boff = 0;
    dst = trunk_keys + ((int64_t)t * hkv + g) * di * tg_stride + j;  // dim-major, groups contiguous
    dstride = tg_stride;
  } else {
    const int64_t bs = slot - n_trunk_items;
    const int b = (int)(bs / max_bg), s = (int)(bs % max_bg);
    const int a = branch_anchor[b], w = branch_len[b];
    j = (a + 1) / G + s;
    if (j > (a + w) / G - 1) return;          // not complete at the branch's last row
    base = tree_off[branch_tree[b]];
    anchor = a;
    boff = branch_off[b];
    dst = branch_keys + (bs * hkv + g) * di;
    dstride = 1;
  }
  for (int d = lane; d < di; d += 64) {
    float acc = 0.f;
    for (int i = 0; i < G; ++i) {
      const int p = j * G + i;
      const int row = p <= anchor ? base + p : boff + (p - anchor - 1);
      acc += bf(ki[((int64_t)row * hkv + g) * di + d]);
    }
    dst[d * dstride] = acc / (float)G;
  }
}

// ---------------------------------------------------------------- selection
constexpr int kSelSlots = 16;  // complete groups per lane: at most 1024 per row

__device__ inline float wave_max_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}

__global__ __launch_bounds__(64 * kQsaWaves) void qsa_select_kernel(
    const __bf16 *__restrict__ qi, int32_t hkv, int32_t di, int32_t G, int32_t top_k, int64_t n_rows,
    const int32_t *__restrict__ row_tree, const int32_t *__restrict__ row_branch,
    const int32_t *__restrict__ row_anchor, const int32_t *__restrict__ row_pos, int32_t tg_stride, int32_t max_bg,
    const float *__restrict__ trunk_keys, const float *__restrict__ branch_keys, int32_t *__restrict__ sel) {
  __shared__ float qs[kQsaWaves][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // workgroup -> (KV head, 4 consecutive rows): consecutive workgroups go to
  // different XCDs, so each XCD's L2 serves one KV head's keys
  const int g = blockIdx.x % hkv;
  const int64_t r0 = (int64_t)(blockIdx.x / hkv) * kQsaWaves + wv;
  const bool live = r0 < n_rows;
  const int64_t r = live ? r0 : 0;
  for (int d = lane; d < di; d += 64) qs[wv][d] = bf(qi[(r * hkv + g) * di + d]);
  __syncthreads();
  if (!live) return;
  const int t = row_pos[r];
  const int n_c = (t + 1) / G;
  const int b = row_branch[r];
  const int jb = b >= 0 ? (row_anchor[r] + 1) / G : n_c;  // first group keyed by the branch
  const int tree = row_tree[r];
  float sc[kSelSlots];
#pragma unroll
  for (int s = 0; s < kSelSlots; ++s) {
    const int j = lane + 64 * s;
    sc[s] = -INFINITY;
    if (j < n_c) {
      // trunk keys are dim-major with the groups contiguous, so the lanes of a
      // wave (consecutive groups) read one dim of 64 keys in one coalesced load
      const bool trunk = j < jb;
      const float *key = trunk ? trunk_keys + ((int64_t)tree * hkv + g) * di * tg_stride + j
                               : branch_keys + (((int64_t)b * max_bg + (j - jb)) * hkv + g) * di;
      const int64_t ks = trunk ? tg_stride : 1;
      float acc = 0.f;
      for (int d = 0; d < di; ++d) acc = fmaf(qs[wv][d], key[d * ks], acc);
      sc[s] = acc;
    }
  }
  // k rounds of a wave arg-max (highest score, then lowest group index)
  uint32_t picked = 0;
  const int kk = min(top_k, n_c);
  for (int it = 0; it < kk; ++it) {
    float best = -INFINITY;
    int bj = INT32_MAX;
#pragma unroll
    for (int s = 0; s < kSelSlots; ++s) {
      const int j = lane + 64 * s;
      const bool ok = j < n_c && !((picked >> s) & 1u);
      if (ok && (sc[s] > best || (sc[s] == best && j < bj))) {
        best = sc[s];
        bj = j;
      }
    }
    const float m = wave_max_f(best);
    const int jw = wave_min_i(best == m ? bj : INT32_MAX);
    if ((jw & 63) == lane) picked |= 1u << (jw >> 6);
  }
  // ascending order: group j = lane + 64 s sits after every pick of an earlier
  // slot and of a lower lane in the same slot
  int32_t *out = sel + (r * hkv + g) * top_k;
  int before = 0;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int s = 0; s < kSelSlots; ++s) {
    const uint64_t m = __ballot((picked >> s) & 1u);
    if ((picked >> s) & 1u) out[before + __popcll(m & below)] = lane + 64 * s;
    before += __popcll(m);
  }
  for (int i = kk + lane; i < top_k; i += 64) out[i] = -1;
}

// ---------------------------------------------------------------- attention
// Key of position i (0..7) of the lane's column group q in half h of a 64-key
// tile, as the V^T tiles store them: chunk c = 4h + q holds keys of the quads
// [0, 2] (c even) or [1, 3] (c odd) of 16-key group c / 2.
__device__ inline int half_key(int h, int q, int i) {
  const int c = 4 * h + q;
  return 16 * (c >> 1) + 4 * (c & 1) + (i & 3) + ((i >> 2) << 3);
}

struct QsaRange {
  int lo, hi;  // packed rows [lo, hi)
};

__global__ __launch_bounds__(64 * kQsaWaves) void qsa_attn_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kt, const __bf16 *__restrict__ vt,
    __bf16 *__restrict__ out, const float2 *__restrict__ tab, int32_t hq, int32_t hkv, int32_t G,
    int32_t top_k, int64_t n_rows, int32_t n_key_tiles, const int32_t *__restrict__ row_tree,
    const int32_t *__restrict__ row_branch, const int32_t *__restrict__ row_anchor,
    const int32_t *__restrict__ row_pos, const int32_t *__restrict__ tree_off,
    const int32_t *__restrict__ branch_off, const int32_t *__restrict__ sel, float sl2) {
  constexpr int D = kQsaD, KS = D / 32, DT = D / 16;
  const int lane = threadIdx.x & 63;
  // workgroup -> (KV head, 4 consecutive rows), as in qsa_select_kernel
  const int g = blockIdx.x % hkv;
  const int64_t r = (int64_t)(blockIdx.x / hkv) * kQsaWaves + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const int grp = hq / hkv;
  const int col = lane & 15, qd = lane >> 4;
  const bool colv = col < grp;

  const int t = row_pos[r];
  const int b = row_branch[r];
  const int a = b >= 0 ? row_anchor[r] : t;  // last trunk position of the history
  const int toff = tree_off[row_tree[r]];
  const int boff = b >= 0 ? branch_off[b] : 0;
  // packed row of history position p
  auto prow = [&](int p) { return p <= a ? toff + p : boff + (p - a - 1); };

  // Q^T fragments: column = query head g*grp + col, dims 32 ks + 8 qd .. + 7,
  // rotated at position t and scaled by scale * log2(e)
  bf16x8 qf[KS];
  {
    const int h = g * grp + (colv ? col : 0);
    const __bf16 *qp = q + (r * hq + h) * D;
    const float2 *tp = tab + (int64_t)t * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = 32 * ks + 8 * qd;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = d0 + e;
        const int j = d < D / 2 ? d : d - D / 2;
        const float2 cs = tp[j];
        const float x1 = bf(qp[j]), x2 = bf(qp[j + D / 2]);
        const float y = d < D / 2 ? x1 * cs.x - x2 * cs.y : x2 * cs.x + x1 * cs.y;
        qf[ks][e] = (__bf16)(colv ? y * sl2 : 0.f);
      }
    }
  }

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const __bf16 *kbase = kt + (int64_t)g * n_key_tiles * kKeyTile * D;
  const __bf16 *vbase = vt + (int64_t)g * n_key_tiles * kKeyTile * D;

  // 32 keys (half h of tile tl) masked to [lo, hi)
  auto half = [&](int tl, int h, int lo, int hi) {
    const __bf16 *kp = kbase + (int64_t)tl * kKeyTile * D;
    const __bf16 *vp = vbase + (int64_t)tl * kKeyTile * D;
    // the V^T fragments go out with the K fragments: both loads of a half are in
    // flight together
    bf16x8 vfr[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 16 * dt + (lane & 15);
      const int c = 4 * h + qd;
      vfr[dt] = *reinterpret_cast<const bf16x8 *>(vp + (d * 8 + (c ^ vt_swizzle(d))) * 8);
    }
    f32x4 s[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      s[x] = f32x4{0.f, 0.f, 0.f, 0.f};
      // A = K rows: row rho = lane & 15 of score tile x holds key half_key(h, rho/4, rho%4 + 4x)
      const int rho = lane & 15;
      const int kr = half_key(h, rho >> 2, (rho & 3) + 4 * x);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = 4 * ks + qd;  // dim chunk
        const bf16x8 af = *reinterpret_cast<const bf16x8 *>(kp + (kr * 16 + (c ^ (kr & 15))) * 8);
        s[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[ks], s[x], 0, 0, 0);
      }
    }
    // the lane's 8 scores: keys half_key(h, qd, i), i = 4x + e
    float p[8];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = tl * kKeyTile + half_key(h, qd, i);
      const float v = (row >= lo && row < hi) ? s[i >> 2][i & 3] : -INFINITY;
      p[i] = v;
      mx = fmaxf(mx, v);
    }
    {
      auto rr = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(rr[0]), __uint_as_float(rr[1]));
      rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(rr[0]), __uint_as_float(rr[1]));
    }
    if (__any(mx > m + kQsaLazyMax)) {
      const float m_new = mx > m + kQsaLazyMax ? mx : m;
      const float corr = m_new == m ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      l *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      m = m_new;
    }
    const float mu = m == -INFINITY ? 0.f : m;
    bf16x8 pf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = __builtin_amdgcn_exp2f(p[i] - mu);
      l += e;
      pf[i] = (__bf16)e;
    }
    // O^T[dims][heads] += V^T[dims][keys] P^T[keys][heads], k-slot 8 qd + i = key half_key(h, qd, i)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr[dt], pf, o[dt], 0, 0, 0);
  };

  // every 32-key half that meets packed rows [lo, hi)
  auto range = [&](int lo, int hi) {
    if (hi <= lo) return;
    for (int h32 = lo >> 5; h32 <= (hi - 1) >> 5; ++h32) half(h32 >> 1, h32 & 1, lo, hi);
  };

  // The picked groups (ascending), then the tail, as history positions; each
  // splits at the anchor into a trunk piece and a branch piece (piece 2i + x),
  // pieces map to packed-row ranges, and ranges that continue each other merge.
  // One loop, one call of `range` (so the tile body is emitted once).
  const int n_c = (t + 1) / G;
  const int kk = min(top_k, n_c);
  const int32_t *ps = sel + (r * hkv + g) * top_k;
  const int n_pieces = 2 * kk + 2;
  int cur_lo = 0, cur_hi = 0;
  for (int idx = 0; idx <= n_pieces; ++idx) {
    int lo = INT32_MAX, hi = INT32_MAX;
    if (idx < n_pieces) {
      const int i = idx >> 1, x = idx & 1;
      int p0, p1;
      if (i < kk) {
        const int j = __builtin_amdgcn_readfirstlane(ps[i]);
        p0 = j * G;
        p1 = j * G + G - 1;
      } else {
        p0 = n_c * G;
        p1 = t;
      }
      if (x == 0) {
        p1 = min(p1, a);
      } else {
        p0 = max(p0, a + 1);
      }
      if (p1 < p0) continue;
      lo = prow(p0);
      hi = prow(p1) + 1;
      if (lo == cur_hi) {
        cur_hi = hi;
        continue;
      }
    }
    range(cur_lo, cur_hi);
    cur_lo = lo;
    cur_hi = hi;
  }

  // column sums over the four lane groups of each column
  {
    auto rr = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    l = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
    rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    l = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
  }
  if (colv) {
    const float inv = 1.f / l;
    __bf16 *op = out + (r * hq + g * grp + col) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      __bf16 r4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r4[e] = (__bf16)(o[dt][e] * inv);
      uint2 pk;
      __builtin_memcpy(&pk, r4, 8);
      *reinterpret_cast<uint2 *>(op + 16 * dt + 4 * qd) = pk;
    }
  }
}

}  // namespace

// trunk keys [tree][Hkv][DI][groups padded to a multiple of 64], then branch keys
// [branch][its groups][Hkv][DI]
static int64_t trunk_group_stride(const spec_tree_layout &L, int32_t G) {
  return (L.max_trunk_len / G + 63) / 64 * 64;
}

size_t qsa_keys_floats(const spec_tree_layout &L, int32_t hkv, int32_t di, int32_t G) {
  const int64_t max_bg = L.max_branch_len > 1 ? (L.max_branch_len - 1 + G - 1) / G : 0;
  return (size_t)((int64_t)L.n_trees * trunk_group_stride(L, G) + (int64_t)L.n_branches * max_bg) * hkv * di;
}

hipError_t launch_qsa(const spec_tree_layout &L, int32_t hq, int32_t hkv, int32_t di, int32_t G,
                      int32_t top_k, const void *q, const void *qi, const void *ki, const void *kt,
                      const void *vt, const float2 *tab, float scale, float *keys, int32_t *sel,
                      void *out, hipStream_t s) {
  const int32_t max_tg = L.max_trunk_len / G;
  const int32_t max_bg = L.max_branch_len > 1 ? (L.max_branch_len - 1 + G - 1) / G : 0;
  const int32_t tg_stride = (int32_t)trunk_group_stride(L, G);
  float *trunk_keys = keys;
  float *branch_keys = keys + (int64_t)L.n_trees * tg_stride * hkv * di;
  const int64_t key_items = ((int64_t)L.n_trees * max_tg + (int64_t)L.n_branches * max_bg) * hkv;
  if (key_items > 0) {
    hipLaunchKernelGGL(qsa_keys_kernel, dim3((unsigned)((key_items + kQsaWaves - 1) / kQsaWaves)),
                       dim3(64 * kQsaWaves), 0, s, static_cast<const __bf16 *>(ki), hkv, di, G, L.tree_off,
                       L.tree_trunk_len, L.n_trees, max_tg, L.branch_tree, L.branch_anchor, L.branch_len,
                       L.branch_off, L.n_branches, max_bg, tg_stride, trunk_keys, branch_keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  prof_mark(s, "qsa_keys");
  const int64_t blocks = (L.n_rows + kQsaWaves - 1) / kQsaWaves * hkv;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)blocks;
  hipLaunchKernelGGL(qsa_select_kernel, dim3(grid), dim3(64 * kQsaWaves), 0, s, static_cast<const __bf16 *>(qi),
                     hkv, di, G, top_k, L.n_rows, L.row_tree, L.row_branch, L.row_anchor, L.row_pos, tg_stride,
                     max_bg, trunk_keys, branch_keys, sel);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "qsa_select");
  const int32_t n_key_tiles = (int32_t)((L.n_rows + kKeyTile - 1) / kKeyTile);
  const float sl2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(qsa_attn_kernel, dim3(grid), dim3(64 * kQsaWaves), 0, s, static_cast<const __bf16 *>(q),
                     static_cast<const __bf16 *>(kt), static_cast<const __bf16 *>(vt),
                     static_cast<__bf16 *>(out), tab, hq, hkv, G, top_k, L.n_rows, n_key_tiles, L.row_tree,
                     L.row_branch, L.row_anchor, L.row_pos, L.tree_off, L.branch_off, sel, sl2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "qsa_attn");
  return hipSuccess;
}

}  // namespace spec
