// Indexed GDN state replay for the branch rows of a packed proposal tree.
//
// [SpecOPD paper page, Figure 5]: the trunk runs once and its FP32 GDN state is
// stored every `chunk` tokens. A branch loads the last stored state at or
// before its anchor into registers, runs the trunk tokens between that state
// and the anchor, then its own tokens, one output per token; stored states are
// never written here, and each token's convolution window runs over its
// ancestors. [SpecOPD paper page, Figure 13]: the replayed trunk tokens count as
// GDN work.
//
// Recurrence (gated delta rule, per head; state S is D x D with value rows i
// and key columns j):
//   u_i  = sum_j S_ij k_j
//   S_ij = alpha S_ij + beta (v_i - alpha u_i) k_j
//   o_i  = sum_j S_ij q_j
// Row i of S moves with its own v_i and the token's shared k, q, alpha and
// beta only. So one lane owns one row, in registers, and the update needs no
// cross-lane traffic: a workgroup is one wavefront holding 64 rows (D / 64
// workgroups per branch and head). The same wave builds each token's
// features: for the q and k channels lane and lane + 64 and for its own v row,
// a convolution over the token and its K-1 nearest ancestors, SiLU, then the
// L2 norms of q and k as wave sums; q~ and k~ reach every lane through LDS as
// uniform (broadcast) reads. Along a branch's path the ancestors of a position
// are simply the positions before it: trunk token p for p <= a, then the
// branch's rows in depth order.
//
// The work is fp32 VALU (three D-long row operations per token per lane);
// the only sizable memory traffic is the checkpoint (D * D * 4 bytes per
// branch and head), read once with each load instruction covering 64
// consecutive value rows of one key column (key-major storage).
#include "common.h"
#include "gdn_util.h"

namespace spec {

// the chunkwise trunk pass (gdn_chunk.hip), for chunk <= 64
size_t gdn_chunk_work_bytes(const spec_tree_layout &L, int H, int D, int chunk);
hipError_t launch_gdn_chunked(const spec_tree_layout &L, int H, int D, int K, int chunk, int n_ckpt,
                              const void *xq, const void *xk, const void *xv, const float *taps,
                              const float *alpha, const float *beta, float *ckpt, float *out,
                              void *work, hipStream_t s);
hipError_t launch_gdn_replay_chunked(const spec_tree_layout &L, int H, int D, int K, int chunk,
                                     int n_ckpt, const void *xq, const void *xk, const void *xv,
                                     const float *taps, const float *alpha, const float *beta,
                                     const float *ckpt, const void *work, float *out,
                                     hipStream_t s);

namespace {

using gdn::silu_f;
using gdn::wave_sum;

// 8 consecutive floats of an LDS array, read with two 128-bit loads (the same
// address in every lane: a broadcast)
struct Chunk {
  float v[8];
};
__device__ inline Chunk load_chunk(const float *lds, int at) {
  const float4 x = *reinterpret_cast<const float4 *>(lds + at);
  const float4 y = *reinterpret_cast<const float4 *>(lds + at + 4);
  return Chunk{{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w}};
}

// Lanes per state row: a row of D <= 64 columns sits in one lane; a row of 128
// in two (lanes l and l + 32, 64 columns each), which keeps a lane's share of
// the state, with the rest of the step, within the 256 architectural VGPRs.
template <int D>
struct GdnShape {
  static constexpr int CW = D > 64 ? 64 : D;  // columns per lane
  static constexpr int LPR = D / CW;          // lanes per row
  static constexpr int RPW = 64 / LPR;        // rows per wave (= per workgroup)
  static constexpr int RB = D / RPW;          // workgroups per branch and head
};

// TRUNK: the shared trunk pass instead of the replay. The path is then a
// tree's whole trunk from the zero state (anchor = last trunk token, no branch
// rows), every token's output is written, and the state after every `chunk`
// tokens is stored as a checkpoint (slot 0: the zero state).
template <int D, int K, bool TRUNK>
__device__ __forceinline__ void gdn_path(
    const int32_t *__restrict__ tree_off, const int32_t *__restrict__ tree_trunk_len,
    const int32_t *__restrict__ branch_tree,
    const int32_t *__restrict__ branch_anchor, const int32_t *__restrict__ branch_len,
    const int32_t *__restrict__ branch_off, const __bf16 *__restrict__ xq,
    const __bf16 *__restrict__ xk, const __bf16 *__restrict__ xv, const float *__restrict__ taps,
    const float *__restrict__ alpha, const float *__restrict__ beta, float *__restrict__ ckpt,
    float *__restrict__ out, int H, int chunk, int n_ckpt, int n_pairs) {
  using G = GdnShape<D>;
  constexpr int CW = G::CW, LPR = G::LPR, RPW = G::RPW, RB = G::RB;
  constexpr int CPL = D / 64;  // q and k channels per lane (lane + 64 m)
  __shared__ __attribute__((aligned(16))) float kq[2 * D];  // k~ of the current token, then q~

  const int lane = threadIdx.x;
  // Workgroups are dealt to the 8 XCDs round-robin; the RB row blocks of one
  // (branch, head) pair take ids 8 apart, so they share an XCD and its L2 holds
  // the token inputs they all read. Pairs are padded to a multiple of 8.
  const int x8 = blockIdx.x % 8, y8 = blockIdx.x / 8;
  const int rb = y8 % RB;
  const int pair = x8 + 8 * (y8 / RB);
  if (pair >= n_pairs) return;
  const int h = pair % H;
  int t, a, W, r0, c;
  if (TRUNK) {  // pair = (tree, head)
    t = pair / H;
    a = tree_trunk_len[t] - 1;
    W = 1;
    r0 = 0;
    c = 0;
  } else {  // pair = (branch, head)
    const int b = pair / H;
    W = branch_len[b];
    if (W < 2) return;  // the branch has no rows (workgroup-uniform, before any barrier)
    t = branch_tree[b];
    a = branch_anchor[b];
    r0 = branch_off[b];
    c = (a + 1) / chunk;
  }
  const int off = tree_off[t];
  const int p_end = a + W;  // path positions c*chunk .. a + W - 1
  const int i = rb * RPW + lane % RPW;  // this lane's state row
  const int cb = (lane / RPW) * CW;     // and its first column
  auto row_of = [&](int p) { return p <= a ? off + p : r0 + (p - a - 1); };
  // sum over the lanes of a row
  auto row_sum = [](float x) {
    if (LPR == 1) return x;
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };

  // this lane's columns of row i from checkpoint c (key-major: column j of row i at j*D + i)
  float S[CW];
  // this lane's part of checkpoint slot `slot` of its tree and head
  auto slot_ptr = [&](int slot) {
    return ckpt + (((int64_t)t * n_ckpt + slot) * H + h) * (int64_t)D * D + (int64_t)cb * D + i;
  };
  if (TRUNK) {
    float *cp = slot_ptr(0);
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      S[j] = 0.f;
      cp[(int64_t)j * D] = 0.f;
    }
  } else {
    const float *cp = slot_ptr(c);
#pragma unroll
    for (int j = 0; j < CW; ++j) S[j] = cp[(int64_t)j * D];
  }
  // convolution taps: q and k channels lane + 64 m, v channel i
  float tq[CPL][K], tk[CPL][K], tv[K];
#pragma unroll
  for (int m = 0; m < CPL; ++m)
#pragma unroll
    for (int j = 0; j < K; ++j) {
      tq[m][j] = taps[(((int64_t)0 * H + h) * D + lane + 64 * m) * K + j];
      tk[m][j] = taps[(((int64_t)1 * H + h) * D + lane + 64 * m) * K + j];
    }
#pragma unroll
  for (int j = 0; j < K; ++j) tv[j] = taps[(((int64_t)2 * H + h) * D + i) * K + j];
  const float qscale = 1.f / sqrtf((float)D);

  // Raw (pre-convolution) inputs of path positions p, p-1, .., p-K+1 (slot 0 =
  // p), zero before position 0; each step loads only the next position, one
  // step ahead, together with its gates.
  struct Raw {
    float q[CPL], k[CPL], v;
  };
  auto load_raw = [&](int pp) {
    Raw x;
#pragma unroll
    for (int m = 0; m < CPL; ++m) x.q[m] = x.k[m] = 0.f;
    x.v = 0.f;
    if (pp >= 0 && pp < p_end) {  // wave-uniform
      const int64_t base = ((int64_t)row_of(pp) * H + h) * D;
#pragma unroll
      for (int m = 0; m < CPL; ++m) {
        x.q[m] = (float)xq[base + lane + 64 * m];
        x.k[m] = (float)xk[base + lane + 64 * m];
      }
      x.v = (float)xv[base + i];
    }
    return x;
  };
  const int p0 = c * chunk;
  Raw win[K];  // as of the step before p0 (slot j = position p0 - 1 - j); each step shifts it
#pragma unroll
  for (int j = 0; j + 1 < K; ++j) win[j] = load_raw(p0 - 1 - j);
  Raw nxt = load_raw(p0);
  float n_al = alpha[(int64_t)row_of(p0) * H + h], n_be = beta[(int64_t)row_of(p0) * H + h];

  for (int p = p0; p < p_end; ++p) {
    const int r = row_of(p);
#pragma unroll
    for (int j = K - 1; j > 0; --j) win[j] = win[j - 1];
    win[0] = nxt;
    const float al = n_al, be = n_be;
    if (p + 1 < p_end) {  // the next position's inputs and gates, in flight during this step
      nxt = load_raw(p + 1);
      const int64_t g = (int64_t)row_of(p + 1) * H + h;
      n_al = alpha[g];
      n_be = beta[g];
    }
    // features: the convolution over the window, SiLU, norms
    float aq[CPL], ak[CPL], av = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) aq[m] = ak[m] = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
#pragma unroll
      for (int m = 0; m < CPL; ++m) {
        aq[m] = fmaf(tq[m][j], win[j].q[m], aq[m]);
        ak[m] = fmaf(tk[m][j], win[j].k[m], ak[m]);
      }
      av = fmaf(tv[j], win[j].v, av);
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      aq[m] = silu_f(aq[m]);
      ak[m] = silu_f(ak[m]);
      sq = fmaf(aq[m], aq[m], sq);
      sk = fmaf(ak[m], ak[m], sk);
    }
    av = silu_f(av);
    const float nq = qscale * __builtin_amdgcn_rsqf(wave_sum(sq)), nk = __builtin_amdgcn_rsqf(wave_sum(sk));
    __syncthreads();  // every lane is done reading the previous token's q~, k~
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      kq[lane + 64 * m] = ak[m] * nk;
      kq[D + lane + 64 * m] = aq[m] * nq;
    }
    __syncthreads();
    // The row passes read this lane's columns of k~ (and q~) as LDS broadcasts
    // (one address per row half) in chunks of 8, PD chunks ahead of the FMAs
    // that use them; the scheduling barriers keep the compiler from hoisting
    // every read into registers at once. Row sums keep 8 partial sums, so their
    // FMAs do not wait on one another, then add the row's other lane.
    constexpr int NC = CW / 8, PD = 4, PD2 = 2;  // chunks in flight: one stream, two streams
    float up[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) up[e] = 0.f;
    {
      Chunk ring[PD];
#pragma unroll
      for (int c0 = 0; c0 < PD; ++c0) ring[c0] = load_chunk(kq, cb + 8 * c0);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const Chunk cur = ring[cc % PD];
        if (cc + PD < NC) ring[cc % PD] = load_chunk(kq, cb + 8 * (cc + PD));
#pragma unroll
        for (int e = 0; e < 8; ++e) up[e] = fmaf(S[8 * cc + e], cur.v[e], up[e]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float u = row_sum(((up[0] + up[1]) + (up[2] + up[3])) + ((up[4] + up[5]) + (up[6] + up[7])));
    const float w = be * (av - al * u);
    if (TRUNK || p > a) {  // a branch token (or any trunk-pass token): update and read out
      float op[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) op[e] = 0.f;
      Chunk rk[PD2], rq[PD2];
#pragma unroll
      for (int c0 = 0; c0 < PD2; ++c0) {
        rk[c0] = load_chunk(kq, cb + 8 * c0);
        rq[c0] = load_chunk(kq, D + cb + 8 * c0);
      }
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const Chunk ck = rk[cc % PD2], cq = rq[cc % PD2];
        if (cc + PD2 < NC) {
          rk[cc % PD2] = load_chunk(kq, cb + 8 * (cc + PD2));
          rq[cc % PD2] = load_chunk(kq, D + cb + 8 * (cc + PD2));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          S[8 * cc + e] = fmaf(w, ck.v[e], al * S[8 * cc + e]);
          op[e] = fmaf(S[8 * cc + e], cq.v[e], op[e]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const float o = row_sum(((op[0] + op[1]) + (op[2] + op[3])) + ((op[4] + op[5]) + (op[6] + op[7])));
      if (cb == 0) out[((int64_t)r * H + h) * D + i] = o;
      if (TRUNK && (p + 1) % chunk == 0) {  // state after tokens 0 .. p: checkpoint (p + 1) / chunk
        float *cp = slot_ptr((p + 1) / chunk);
#pragma unroll
        for (int j = 0; j < CW; ++j) cp[(int64_t)j * D] = S[j];
      }
    } else {  // a replayed trunk token: update only
      Chunk ring[PD];
#pragma unroll
      for (int c0 = 0; c0 < PD; ++c0) ring[c0] = load_chunk(kq, cb + 8 * c0);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const Chunk cur = ring[cc % PD];
        if (cc + PD < NC) ring[cc % PD] = load_chunk(kq, cb + 8 * (cc + PD));
#pragma unroll
        for (int e = 0; e < 8; ++e) S[8 * cc + e] = fmaf(w, cur.v[e], al * S[8 * cc + e]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

#define SPEC_GDN_PARAMS                                                                            \
  const int32_t *__restrict__ tree_off, const int32_t *__restrict__ tree_trunk_len,                \
      const int32_t *__restrict__ branch_tree, const int32_t *__restrict__ branch_anchor,          \
      const int32_t *__restrict__ branch_len, const int32_t *__restrict__ branch_off,              \
      const __bf16 *__restrict__ xq, const __bf16 *__restrict__ xk, const __bf16 *__restrict__ xv, \
      const float *__restrict__ taps, const float *__restrict__ alpha,                             \
      const float *__restrict__ beta, float *__restrict__ ckpt, float *__restrict__ out, int H,    \
      int chunk, int n_ckpt, int n_pairs
#define SPEC_GDN_ARGS                                                                         \
  tree_off, tree_trunk_len, branch_tree, branch_anchor, branch_len, branch_off, xq, xk, xv, \
      taps, alpha, beta, ckpt, out, H, chunk, n_ckpt, n_pairs

// The trunk pass and the replay as kernels of their own names.
template <int D, int K>
__global__ __launch_bounds__(64) void gdn_trunk_kernel(SPEC_GDN_PARAMS) {
  gdn_path<D, K, true>(SPEC_GDN_ARGS);
}
template <int D, int K>
__global__ __launch_bounds__(64) void gdn_replay_kernel(SPEC_GDN_PARAMS) {
  gdn_path<D, K, false>(SPEC_GDN_ARGS);
}

template <int D, int K, bool TRUNK>
hipError_t launch_gdn(const spec_tree_layout &L, int H, int chunk, int n_ckpt, const void *xq,
                      const void *xk, const void *xv, const float *taps, const float *alpha,
                      const float *beta, float *ckpt, float *out, hipStream_t s) {
  const int64_t pairs = (int64_t)(TRUNK ? L.n_trees : L.n_branches) * H;
  const int64_t blocks = (pairs + 7) / 8 * 8 * GdnShape<D>::RB;
  if (pairs == 0) return hipSuccess;
  auto kern = TRUNK ? gdn_trunk_kernel<D, K> : gdn_replay_kernel<D, K>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64), 0, s, L.tree_off, L.tree_trunk_len,
                     L.branch_tree, L.branch_anchor, L.branch_len, L.branch_off,
                     static_cast<const __bf16 *>(xq), static_cast<const __bf16 *>(xk),
                     static_cast<const __bf16 *>(xv), taps, alpha, beta, ckpt, out, H, chunk, n_ckpt,
                     (int)pairs);
  return hipGetLastError();
}

template <int D, bool TRUNK>
hipError_t launch_gdn_d(int K, const spec_tree_layout &L, int H, int chunk, int n_ckpt,
                        const void *xq, const void *xk, const void *xv, const float *taps,
                        const float *alpha, const float *beta, float *ckpt, float *out,
                        hipStream_t s) {
  switch (K) {
    case 1: return launch_gdn<D, 1, TRUNK>(L, H, chunk, n_ckpt, xq, xk, xv, taps, alpha, beta, ckpt, out, s);
    case 2: return launch_gdn<D, 2, TRUNK>(L, H, chunk, n_ckpt, xq, xk, xv, taps, alpha, beta, ckpt, out, s);
    case 3: return launch_gdn<D, 3, TRUNK>(L, H, chunk, n_ckpt, xq, xk, xv, taps, alpha, beta, ckpt, out, s);
    case 4: return launch_gdn<D, 4, TRUNK>(L, H, chunk, n_ckpt, xq, xk, xv, taps, alpha, beta, ckpt, out, s);
  }
  return hipErrorInvalidValue;
}

// Argument checks shared by the trunk pass and the replay.
spec_status check_gdn(const spec_tree_layout *layout, bool trunk, int32_t n_heads, int32_t head_dim,
                      int32_t conv_width, int32_t chunk, const void *const *bufs, int n_bufs) {
  if (!layout) return fail(SPEC_ERR_INVALID_ARG, "layout must be non-NULL");
  const spec_tree_layout &L = *layout;
  if (L.n_trees < 1 || L.n_rows < 1 || L.n_branches < 0 || L.max_trunk_len < 1)
    return fail(SPEC_ERR_INVALID_ARG, "layout scalars are not those of a packed tree");
  const bool need = trunk ? true : L.n_branches > 0;
  if (need && (!L.tree_off || (trunk && !L.tree_trunk_len) ||
               (!trunk && (!L.branch_tree || !L.branch_anchor || !L.branch_len || !L.branch_off))))
    return fail(SPEC_ERR_INVALID_ARG, "layout device arrays are missing (pack with a buffer first)");
  if (n_heads < 1) return fail(SPEC_ERR_INVALID_ARG, "n_heads must be >= 1 (got %d)", n_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(SPEC_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (conv_width < 1 || conv_width > 4)
    return fail(SPEC_ERR_UNSUPPORTED, "conv_width %d not in 1..4", conv_width);
  if (chunk < 1) return fail(SPEC_ERR_INVALID_ARG, "chunk must be >= 1 (got %d)", chunk);
  const int64_t pairs = (int64_t)(trunk ? L.n_trees : L.n_branches) * n_heads;
  if ((pairs + 7) / 8 * 8 * (head_dim / 32) > INT32_MAX)
    return fail(SPEC_ERR_UNSUPPORTED, "too many %s x heads", trunk ? "trees" : "branches");
  for (int k = 0; k < n_bufs; ++k)
    if (!bufs[k]) return fail(SPEC_ERR_INVALID_ARG, "device buffers must be non-NULL");
  for (int k = 0; k < n_bufs; ++k)
    if (!aligned16(bufs[k])) return fail(SPEC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  return SPEC_OK;
}

spec_status run_gdn(bool trunk, const spec_tree_layout *layout, int32_t n_heads, int32_t head_dim,
                    int32_t conv_width, int32_t chunk, const void *d_xq, const void *d_xk,
                    const void *d_xv, const float *d_taps, const float *d_alpha, const float *d_beta,
                    float *d_ckpt, float *d_out, void *d_work, size_t *work_bytes, spec_stream stream,
                    const void *d_trunk_work = nullptr) {
  clear_error();
  if (trunk && !work_bytes) return fail(SPEC_ERR_INVALID_ARG, "work_bytes must be non-NULL");
  if (trunk && !d_work) {  // size query
    if (!layout) return fail(SPEC_ERR_INVALID_ARG, "layout must be non-NULL");
    if (chunk < 1) return fail(SPEC_ERR_INVALID_ARG, "chunk must be >= 1 (got %d)", chunk);
    if (n_heads < 1 || (head_dim != 64 && head_dim != 128))
      return fail(SPEC_ERR_INVALID_ARG, "need n_heads >= 1 and head_dim in {64, 128}");
    *work_bytes = gdn_chunk_work_bytes(*layout, n_heads, head_dim, chunk);
    return SPEC_OK;
  }
  const void *bufs[] = {d_xq, d_xk, d_xv, d_taps, d_alpha, d_beta, d_ckpt, d_out};
  spec_status st = check_gdn(layout, trunk, n_heads, head_dim, conv_width, chunk, bufs, 8);
  if (st != SPEC_OK) return st;
  const spec_tree_layout &L = *layout;
  const int n_ckpt = L.max_trunk_len / chunk + 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (trunk) {
    const size_t need = gdn_chunk_work_bytes(L, n_heads, head_dim, chunk);
    if (*work_bytes < need) {
      const size_t have = *work_bytes;
      *work_bytes = need;
      return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    }
    if (!aligned16(d_work)) return fail(SPEC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  }
  if (trunk && chunk <= 64) {
    if ((int64_t)L.n_trees * ((L.max_trunk_len + chunk - 1) / chunk) * n_heads > INT32_MAX)
      return fail(SPEC_ERR_UNSUPPORTED, "too many trees x chunks x heads");
    prof_mark(s, "gdn_trunk:begin");
    const hipError_t e = launch_gdn_chunked(L, n_heads, head_dim, conv_width, chunk, n_ckpt, d_xq, d_xk,
                                            d_xv, d_taps, d_alpha, d_beta, d_ckpt, d_out, d_work, s);
    if (e != hipSuccess) return hip_fail(e, "chunkwise GDN trunk pass launch");
    return SPEC_OK;
  }
  if (!trunk && d_trunk_work) {  // the replay from the trunk pass's cache
    if (chunk > 64)
      return fail(SPEC_ERR_INVALID_ARG, "a trunk-pass cache exists only for chunk <= 64 (got %d)", chunk);
    if (!aligned16(d_trunk_work)) return fail(SPEC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    if (L.max_branch_len > 65) return fail(SPEC_ERR_UNSUPPORTED, "branches longer than 65 tokens");
    if (!L.branch_order) return fail(SPEC_ERR_INVALID_ARG, "layout device arrays are missing");
    prof_mark(s, "gdn:begin");
    const hipError_t e = launch_gdn_replay_chunked(L, n_heads, head_dim, conv_width, chunk, n_ckpt, d_xq,
                                                   d_xk, d_xv, d_taps, d_alpha, d_beta, d_ckpt,
                                                   d_trunk_work, d_out, s);
    if (e != hipSuccess) return hip_fail(e, "gdn_replay_chunk_kernel launch");
    prof_mark(s, "gdn_replay_chunk");
    return SPEC_OK;
  }
  prof_mark(s, trunk ? "gdn_trunk:begin" : "gdn:begin");
  hipError_t e;
  if (trunk)
    e = head_dim == 64 ? launch_gdn_d<64, true>(conv_width, L, n_heads, chunk, n_ckpt, d_xq, d_xk, d_xv,
                                                d_taps, d_alpha, d_beta, d_ckpt, d_out, s)
                       : launch_gdn_d<128, true>(conv_width, L, n_heads, chunk, n_ckpt, d_xq, d_xk,
                                                 d_xv, d_taps, d_alpha, d_beta, d_ckpt, d_out, s);
  else
    e = head_dim == 64 ? launch_gdn_d<64, false>(conv_width, L, n_heads, chunk, n_ckpt, d_xq, d_xk,
                                                 d_xv, d_taps, d_alpha, d_beta, d_ckpt, d_out, s)
                       : launch_gdn_d<128, false>(conv_width, L, n_heads, chunk, n_ckpt, d_xq, d_xk,
                                                  d_xv, d_taps, d_alpha, d_beta, d_ckpt, d_out, s);
  if (e != hipSuccess) return hip_fail(e, trunk ? "gdn_trunk_kernel launch" : "gdn_replay_kernel launch");
  prof_mark(s, trunk ? "gdn_trunk" : "gdn_replay");
  return SPEC_OK;
}

}  // namespace

}  // namespace spec

using namespace spec;

extern "C" spec_status spec_gdn_replay_fwd(const spec_tree_layout *layout, int32_t n_heads,
                                           int32_t head_dim, int32_t conv_width, int32_t chunk,
                                           const void *d_xq, const void *d_xk, const void *d_xv,
                                           const float *d_taps, const float *d_alpha,
                                           const float *d_beta, const float *d_ckpt,
                                           const void *d_trunk_work, float *d_out,
                                           spec_stream stream) {
  // the replay only reads the checkpoints (and the trunk pass's cache)
  return run_gdn(false, layout, n_heads, head_dim, conv_width, chunk, d_xq, d_xk, d_xv, d_taps, d_alpha,
                 d_beta, const_cast<float *>(d_ckpt), d_out, nullptr, nullptr, stream, d_trunk_work);
}

extern "C" spec_status spec_gdn_trunk_fwd(const spec_tree_layout *layout, int32_t n_heads,
                                          int32_t head_dim, int32_t conv_width, int32_t chunk,
                                          const void *d_xq, const void *d_xk, const void *d_xv,
                                          const float *d_taps, const float *d_alpha,
                                          const float *d_beta, float *d_ckpt, float *d_out,
                                          void *d_work, size_t *work_bytes, spec_stream stream) {
  return run_gdn(true, layout, n_heads, head_dim, conv_width, chunk, d_xq, d_xk, d_xv, d_taps, d_alpha,
                 d_beta, d_ckpt, d_out, d_work, work_bytes, stream);
}
