// Chunkwise shared trunk pass of GDN scoring.
//
// [SpecOPD paper page, Figure 5]: the shared trunk pass keeps an FP32 GDN
// state at every `chunk`-token boundary of the trunk; the branches replay from
// those states. This file computes that pass a chunk at a time instead of a
// token at a time, with the same result up to rounding.
//
// Recurrence (per head; S is D x D with value rows and key columns):
//   S_s = alpha_s S_{s-1} + delta_s k_s^T,  delta_s = beta_s (v_s - alpha_s S_{s-1} k_s),
//   o_s = S_s q_s.
// Take one chunk of L <= 64 trunk tokens that starts from state S0, and let
// g_s be the running sum of log alpha over the chunk's tokens 0..s. Unrolling
// the recurrence inside the chunk gives
//   delta_s = beta_s (v_s - e^{g_s} S0 k_s - sum_{r<s} e^{g_s - g_r} (k_s.k_r) delta_r),
// a lower-triangular system, so delta = U - W S0^T with
//   [U | W] = (I + diag(beta) A)^{-1} diag(beta) [V | e^{g} K],  A_sr = e^{g_s-g_r} k_s.k_r (r < s).
// Then, with P_sr = e^{g_s-g_r} q_s.k_r (r <= s),
//   o     = (e^{g} Q - P W) S0^T + P U                = Q' S0^T + O'
//   S_end = e^{g_{L-1}} S0 + sum_r e^{g_{L-1}-g_r} delta_r k_r^T = gamma S0 + delta^T Kd.
// Everything except the last line is independent of S0, so it runs for all
// chunks at once; only S_end chains the chunks. Three kernels:
//   prep (tree, chunk, head): features of the chunk's tokens (convolution along
//        the trunk, SiLU, L2 norms), A and P, the triangular solve, Q', O', Kd.
//   scan (tree, head, 16 value rows): delta = U - W S^T and S <- gamma S +
//        delta^T Kd over the chunks in order on the fp32 matrix cores, storing
//        each full chunk's end state as the next checkpoint (and every chunk's
//        delta, a last partial one included, for the replay).
//   out  (tree, chunk, head): o = Q' S_c^T + O' from checkpoint c, on the
//        fp32 matrix cores.
// A chunk tile always has 64 rows; rows past the chunk's tokens are zero.
// Intermediates live in a caller-provided workspace, which also keeps, per
// chunk, the deltas, the normalised keys and g for the branch replay below.
//
// Branch replay from that cache ([SpecOPD paper page, Figure 5]: a branch
// copies the checkpoint at or below its anchor a, replays the trunk tokens
// after it through a, then takes its own tokens). With c = floor((a+1)/C) and
// j = a + 1 - cC replayed tokens of chunk c, the state after the anchor is
//   S_a = e^{G} S_c + sum_{r<j} e^{G - g_r} delta_r k_r^T,   G = g_{j-1},
// where delta_r are chunk c's own deltas (delta_r depends only on S_c and the
// chunk's tokens up to r, so the first j of them are the replayed tokens' updates).
// The branch's m = W - 1 tokens are one more chunk that starts from S_a: with
// its Q', O' from the same in-chunk algebra, its outputs are
//   o = Q' S_a^T + O' = e^{G} Q' S_c^T + (Q' K'^T) Delta + O',  K'_r = e^{G - g_r} k_r,
// three small products on the fp32 matrix cores; S_a is never formed. One
// workgroup per (branch, head) does it all (gdn_replay_chunk_kernel).
#include "common.h"
#include "gdn_util.h"

namespace spec {

namespace {

using gdn::silu_f;
using gdn::wave_sum;

constexpr int CT = 64;    // rows of a chunk tile (the chunk length is at most this)
constexpr int NREC = 7;   // per (tree, chunk, head): W, U, Kd, Q', O', delta, k~; each CT x D
enum { RW = 0, RU = 1, RKD = 2, RQ = 3, RO = 4, RDL = 5, RKF = 6 };

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ inline f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// (s_waitcnt lgkmcnt(0); vmcnt and expcnt left at their maxima), then
// s_barrier. __syncthreads() would also wait for every global load and store
// in flight, which would drain loads issued for a later phase. No kernel here
// passes data between waves through global memory.
constexpr int kWaitLgkm0 = 0xC07F;
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__device__ inline float *rec_part(float *ws, int64_t item, int part) {
  return ws + (item * NREC + part) * (int64_t)(CT * D);
}
template <int D>
__device__ inline const float *rec_part(const float *ws, int64_t item, int part) {
  return ws + (item * NREC + part) * (int64_t)(CT * D);
}

// ---------------------------------------------------------------------------
// The in-chunk algebra shared by the trunk prep and the branch replay: MT rows
// (16, 32 or 64), 256 threads.
// The arrays that unrolled code reads at many fixed offsets come first, so
// that their addresses fit the 16-bit offset field of an LDS instruction.
template <int D, int MT>
struct ChunkLds {
  float Al[MT][MT + 4];
  float Pl[MT][MT + 4];
  float g[64], eg[64], bt[64];  // running log decay, its exponential, beta
  float nk[MT], nq[MT];
  float kf[MT][D + 4];  // k~ (padded rows: 16 consecutive rows start 4 banks apart)
  float qf[MT][D + 4];  // q~
  float vf[MT][D + 4];  // v~ (padded like k~, so a column has one stride)
};

// Features of the tile's tokens: token s is path position P0 + s (s < L), the
// convolution reads positions P0 + s - j, and row_of maps a position to its
// packed row. Thread (d, group) takes channel d of MT / G consecutive tokens;
// the raw rows they read (K - 1 more before the first) are loaded in one batch.
// Then the gates (a wave scan of log alpha; alpha = 1, beta = 0 past L), the
// norms, and k~ and q~ scaled in place. Ends with a barrier.
template <int D, int K, int MT, class RowOf>
__device__ __forceinline__ void chunk_features(ChunkLds<D, MT> &sm, RowOf row_of, int P0, int L,
                                      const __bf16 *__restrict__ xq, const __bf16 *__restrict__ xk,
                                      const __bf16 *__restrict__ xv, const float *__restrict__ taps,
                                      const float *__restrict__ alpha,
                                      const float *__restrict__ beta, int H, int h) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float la = 0.f, b = 0.f;  // this lane's gates (wave 0), loaded first
  if (wv == 0 && lane < L) {
    const int64_t gi = (int64_t)row_of(P0 + lane) * H + h;
    la = alpha[gi];
    b = beta[gi];
  }
  {
    constexpr int G = 256 / D, TPG = MT / G, NR = TPG + K - 1;
    const int d = tid % D, s0 = (tid / D) * TPG;
    float tq[K], tk[K], tv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      tq[j] = taps[(((int64_t)0 * H + h) * D + d) * K + j];
      tk[j] = taps[(((int64_t)1 * H + h) * D + d) * K + j];
      tv[j] = taps[(((int64_t)2 * H + h) * D + d) * K + j];
    }
    float rq[NR], rk[NR], rv[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {  // raw row i is position P0 + s0 - (K - 1) + i
      const int p = P0 + s0 - (K - 1) + i;
      const bool ok = p >= 0 && p < P0 + L;
      const int64_t at = ((int64_t)row_of(ok ? p : P0) * H + h) * D + d;
      const float q = (float)xq[at], k = (float)xk[at], v = (float)xv[at];
      rq[i] = ok ? q : 0.f;
      rk[i] = ok ? k : 0.f;
      rv[i] = ok ? v : 0.f;
    }
#pragma unroll
    for (int s = 0; s < TPG; ++s) {
      float aq = 0.f, ak = 0.f, av = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) {  // tap j reads position P0 + s0 + s - j
        aq = fmaf(tq[j], rq[s + K - 1 - j], aq);
        ak = fmaf(tk[j], rk[s + K - 1 - j], ak);
        av = fmaf(tv[j], rv[s + K - 1 - j], av);
      }
      const bool live = s0 + s < L;
      sm.qf[s0 + s][d] = live ? silu_f(aq) : 0.f;
      sm.kf[s0 + s][d] = live ? silu_f(ak) : 0.f;
      sm.vf[s0 + s][d] = live ? silu_f(av) : 0.f;
    }
  }
  if (wv == 0) {
    la = lane < L ? __logf(la) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(la, o);
      if (lane >= o) la += y;
    }
    sm.g[lane] = la;
    sm.eg[lane] = __expf(la);
    sm.bt[lane] = b;
  }
  lds_barrier();
  const float qscale = 1.f / sqrtf((float)D);
  for (int s = wv; s < MT; s += 4) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int d = lane; d < D; d += 64) {
      sk = fmaf(sm.kf[s][d], sm.kf[s][d], sk);
      sq = fmaf(sm.qf[s][d], sm.qf[s][d], sq);
    }
    sk = wave_sum(sk);
    sq = wave_sum(sq);
    if (lane == 0) {
      sm.nk[s] = s < L ? __builtin_amdgcn_rsqf(sk) : 0.f;
      sm.nq[s] = s < L ? qscale * __builtin_amdgcn_rsqf(sq) : 0.f;
    }
  }
  lds_barrier();
  for (int i = tid; i < MT * D; i += 256) {
    const int s = i / D, d = i % D;
    sm.kf[s][d] *= sm.nk[s];
    sm.qf[s][d] *= sm.nq[s];
  }
  lds_barrier();
}

// A_sr = e^{g_s-g_r} k_s.k_r (r < s) and P_sr = e^{g_s-g_r} q_s.k_r (r <= s) as
// 16 x 16 tiles on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): the tiles on
// and below the diagonal of A, then of P, dealt to the 4 waves in turn; K runs
// over the D feature columns, lane group g taking columns g D/4 .. (g+1) D/4 - 1,
// so each lane reads its rows of k~ (or q~) and k~ as 128-bit LDS loads. Tiles
// above the diagonal are never read by the solve and are left alone. Ends with
// a barrier.
template <int D, int MT>
__device__ __forceinline__ void chunk_ap(ChunkLds<D, MT> &sm) {
  constexpr int NT = MT / 16, TRI = NT * (NT + 1) / 2, KG = D / 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  for (int tix = w; tix < 2 * TRI; tix += 4) {  // uniform per wave
    const bool isp = tix >= TRI;
    int k = isp ? tix - TRI : tix, si = 0;
    while (k > si) k -= ++si;  // lower-triangle tile (si, ri = k)
    const int ri = k;
    const float *xs = isp ? &sm.qf[16 * si + c][g * KG] : &sm.kf[16 * si + c][g * KG];
    const float *xr = &sm.kf[16 * ri + c][g * KG];
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KG / 4; ++i) {
      const float4 a4 = ld4(xs + 4 * i), b4 = ld4(xr + 4 * i);
      acc0 = mfma4(a4.x, b4.x, acc0);
      acc1 = mfma4(a4.y, b4.y, acc1);
      acc0 = mfma4(a4.z, b4.z, acc0);
      acc1 = mfma4(a4.w, b4.w, acc1);
    }
    const f32x4 acc = acc0 + acc1;  // row 16 si + 4g + e, column 16 ri + c
    const int r = 16 * ri + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 16 * si + 4 * g + e;
      const float v = __expf(sm.g[s] - sm.g[r]) * acc[e];  // kept only where r <= s, so e^.. <= 1
      if (isp) sm.Pl[s][r] = r <= s ? v : 0.f;
      else sm.Al[s][r] = r < s ? v : 0.f;
    }
  }
  lds_barrier();
}

// The triangular solve for [U | W] and P [U | W], one column per thread:
// thread j < D takes column j of U, thread D + j column j of W (rows of A and
// P are LDS broadcasts). For each row s, epi_x(s, x) receives the thread's
// entry x of U or W, then epi_y(s, val) receives val = O'[s][j] = (P U)[s][j]
// or Q'[s][j] = e^{g_s} q_s[j] - (P W)[s][j]. Each thread touches only its own
// column of vf (U threads) or of kf and qf (W threads), so epi may overwrite that
// column of vf or qf. With WITH_Y false the P product is left out and the
// thread's column of [U | W] is written back over its right-hand-side column
// (for chunk_px_mfma). Threads 2D and up return at once.
template <int D, int MT, bool WITH_Y = true, class EpiX, class EpiY>
__device__ __forceinline__ void chunk_solve(ChunkLds<D, MT> &sm, EpiX epi_x, EpiY epi_y) {
  const int j = threadIdx.x;
  if (j >= 2 * D) return;
  // column j of the right-hand side: v (j < D) or e^g k; branch-free so the
  // whole solve stays one scheduling region
  const bool isv = j < D;
  const int col = isv ? j : j - D;
  const float *rhs = isv ? &sm.vf[0][col] : &sm.kf[0][col];
  const float *qcol = isv ? &sm.kf[0][0] : &sm.qf[0][col];  // read only for W columns
  float x[MT];
#pragma unroll
  for (int s = 0; s < MT; ++s) x[s] = 0.f;
#pragma unroll
  for (int s = 0; s < MT; ++s) {
    // short tiles: two accumulation chains (even and odd groups of four), so a
    // row's sum waits on half as many dependent FMAs (the 64-row tile keeps one:
    // it has enough independent work and schedules better that way)
    float acc = rhs[s * (D + 4)] * (isv ? 1.f : sm.eg[s]), acc2 = 0.f;
#pragma unroll
    for (int r0 = 0; r0 < s; r0 += 4) {  // A_sr = 0 and x_r = 0 for r >= s
      const float4 a = ld4(&sm.Al[s][r0]);
      float &ac = (MT < 64 && (r0 & 4)) ? acc2 : acc;
      ac = fmaf(-a.x, x[r0], ac);
      ac = fmaf(-a.y, x[r0 + 1], ac);
      ac = fmaf(-a.z, x[r0 + 2], ac);
      ac = fmaf(-a.w, x[r0 + 3], ac);
    }
    x[s] = sm.bt[s] * (acc + acc2);
    if (s % 8 == 7) __builtin_amdgcn_sched_barrier(0);  // bounds how far reads are hoisted
  }
#pragma unroll
  for (int s = 0; s < MT; ++s) epi_x(s, x[s]);
  if (!WITH_Y) {  // x back into this thread's own right-hand-side column, for chunk_px_mfma
    float *xc = const_cast<float *>(rhs);
#pragma unroll
    for (int s = 0; s < MT; ++s) xc[s * (D + 4)] = x[s];
    return;
  }
#pragma unroll
  for (int s = 0; s < MT; ++s) {
    float acc = 0.f, acc2 = 0.f;
#pragma unroll
    for (int r0 = 0; r0 <= s; r0 += 4) {  // P_sr = 0 for r > s
      const float4 p = ld4(&sm.Pl[s][r0]);
      float &ac = (MT < 64 && (r0 & 4)) ? acc2 : acc;
      ac = fmaf(p.x, x[r0], ac);
      ac = fmaf(p.y, x[r0 + 1], ac);
      ac = fmaf(p.z, x[r0 + 2], ac);
      ac = fmaf(p.w, x[r0 + 3], ac);
    }
    acc += acc2;
    const float qv = qcol[s * (D + 4)];
    epi_y(s, isv ? acc : sm.eg[s] * qv - acc);
    if (s % 8 == 7) __builtin_amdgcn_sched_barrier(0);
  }
}

// P [U | W] on the fp32 matrix cores, for the 64-row tile after chunk_solve<...,
// false> has put [U | W] into the right-hand-side columns (U over v~, W over k~).
// Output tiles of 16 rows x 16 columns, 16 per wave (wave w: columns 64w ..
// 64w + 63, all in U or all in W); only the K blocks at or below the tile's rows
// (P is lower-triangular). epi(s, col, isv, val) receives O'[s][col] or
// Q'[s][col] = e^{g_s} q_s[col] - (P W)[s][col]. Starts with a barrier.
template <int D, class Epi>
__device__ __forceinline__ void chunk_px_mfma(ChunkLds<D, CT> &sm, Epi epi) {
  lds_barrier();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  constexpr int NTW = 2 * D / 16 / 4;  // 16-column tiles per wave
#pragma unroll 1
  for (int q = 0; q < NTW; ++q) {
    const int col0 = 16 * (NTW * w + q);  // first of the tile's 2D columns
    const bool isv = col0 < D;
    const int cb = isv ? col0 : col0 - D;
    const float *X = isv ? &sm.vf[0][cb + c] : &sm.kf[0][cb + c];
#pragma unroll
    for (int mt = 0; mt < CT / 16; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4 * (mt + 1); ++st) {  // K rows r = 4 st + g <= 16 mt + 15
        const int r = 4 * st + g;
        acc = mfma4(sm.Pl[16 * mt + c][r], X[r * (D + 4)], acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int srow = 16 * mt + 4 * g + e;
        const float y = acc[e];
        epi(srow, cb + c, isv, isv ? y : sm.eg[srow] * sm.qf[srow][cb + c] - y);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// prep: one workgroup of 256 per (tree, chunk, head), item = (t * n_chunks + c) * H + h.
template <int D, int K>
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(
    const int32_t *__restrict__ tree_off, const int32_t *__restrict__ tree_trunk_len,
    const __bf16 *__restrict__ xq, const __bf16 *__restrict__ xk, const __bf16 *__restrict__ xv,
    const float *__restrict__ taps, const float *__restrict__ alpha,
    const float *__restrict__ beta, float *__restrict__ ws, float *__restrict__ gam,
    float *__restrict__ glog, int H, int chunk, int n_chunks) {
  __shared__ __attribute__((aligned(16))) ChunkLds<D, CT> sm;
  const int64_t item = blockIdx.x;
  const int h = (int)(item % H);
  const int c = (int)((item / H) % n_chunks);
  const int t = (int)(item / ((int64_t)H * n_chunks));
  const int T = tree_trunk_len[t];
  const int p0 = c * chunk;  // trunk position of the tile's row 0
  if (p0 >= T) return;       // workgroup-uniform, before any barrier
  const int L = min(chunk, T - p0);
  const int off = tree_off[t];
  const int tid = threadIdx.x;

  chunk_features<D, K, CT>(sm, [&](int p) { return off + p; }, p0, L, xq, xk, xv, taps, alpha,
                           beta, H, h);
  chunk_ap<D, CT>(sm);
  // Kd_s = e^{g_{L-1} - g_s} k_s (g is flat past L, so g[CT-1] = g[L-1]), stored
  // key-major; k~ row-major and g, for the branch replay. Before the solve, which
  // puts W over k~; the barrier keeps every read of k~ ahead of that.
  {
    float *kd = rec_part<D>(ws, item, RKD);
    float *kt = rec_part<D>(ws, item, RKF);
    const float gl = sm.g[CT - 1];
    for (int i = tid; i < CT * D; i += 256) {
      const int key = i / CT, s = i % CT;
      kd[i] = __expf(gl - sm.g[s]) * sm.kf[s][key];
      kt[i] = sm.kf[i / D][i % D];
    }
  }
  if (tid < CT) glog[item * CT + tid] = sm.g[tid];
  lds_barrier();
  {
    const bool isv = tid < D;
    const int col = isv ? tid : tid - D;
    float *dx = rec_part<D>(ws, item, isv ? RU : RW) + col;  // U or W
    chunk_solve<D, CT, false>(sm, [&](int s, float x) { dx[s * D] = x; }, [](int, float) {});
  }
  {
    float *ro = rec_part<D>(ws, item, RO), *rq = rec_part<D>(ws, item, RQ);
    chunk_px_mfma<D>(sm, [&](int s, int col, bool isv, float val) { (isv ? ro : rq)[s * D + col] = val; });
  }
  if (tid == 0) gam[item] = sm.eg[CT - 1];
}

// ---------------------------------------------------------------------------
// scan: one workgroup of 256 per (tree, head, 16 value rows), on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds C[4 (l / 16) + r][l % 16], r = 0..3). Per chunk:
//   delta (64 tokens x 16 rows) = U - W S^T: wave w takes tokens 16w..16w+15,
//        K runs over the keys, lane group g taking keys g D/4 .. (g+1) D/4 - 1;
//   S (16 rows x D keys) = gamma S + delta^T Kd: wave w owns D/64 tiles of 16
//        keys in registers, K runs over the tokens, group g taking 16g .. 16g+15.
// W, Kd (stored key-major) and the block's U columns are read with coalesced
// loads one chunk ahead into registers, then written to LDS, from which the
// matrix operands are read (a lane's operands lie in 16 rows of W or Kd, which
// straight from memory would touch a new cache line per lane). delta and S
// pass between waves through LDS. delta goes to the workspace for the branch
// replay, also for a last partial chunk (whose end state is not needed). The
// D / 16 row blocks of one (tree, head) take workgroup ids 8 apart, so they
// run on one XCD and share its L2 for W and Kd.
template <int D>
__global__ __launch_bounds__(256) void gdn_chunk_scan_kernel(
    const int32_t *__restrict__ tree_trunk_len, float *__restrict__ ws,
    const float *__restrict__ gam, float *__restrict__ ckpt, int H, int chunk, int n_chunks,
    int n_ckpt, int n_pairs) {
  constexpr int RB = 16, NB = D / RB;
  constexpr int KW = D / 4;              // keys per lane group in the delta product
  constexpr int NT = D / 64;             // 16-key state tiles per wave
  constexpr int NW4 = CT * D / 4 / 256;  // float4 pieces of a CT x D tile per thread
  __shared__ __attribute__((aligned(16))) float Wl[CT][D + 4];   // W of the chunk
  __shared__ __attribute__((aligned(16))) float Kl[D][CT + 4];   // Kd, key-major
  __shared__ __attribute__((aligned(16))) float Ul[CT][RB];      // the block's U columns
  __shared__ __attribute__((aligned(16))) float Sl[RB][D + 4];   // S of the block
  __shared__ __attribute__((aligned(16))) float DlT[RB][CT + 4];  // delta, row-major by value row

  const int x8 = blockIdx.x % 8, y8 = blockIdx.x / 8;
  const int vb = y8 % NB, pair = x8 + 8 * (y8 / NB);
  if (pair >= n_pairs) return;
  const int h = pair % H, t = pair / H;
  const int T = tree_trunk_len[t];
  const int nfull = T / chunk;                // chunks whose end state is a checkpoint
  const int nall = (T + chunk - 1) / chunk;   // chunks whose deltas the replay may read
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  // key-major checkpoint: column k of value row v at k * D + v
  float *ck = ckpt + ((int64_t)t * n_ckpt * H + h) * (int64_t)D * D + vb * RB;
  const int64_t slot_stride = (int64_t)H * D * D;
  f32x4 S[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = tid; i < RB * D; i += 256) Sl[i / D][i % D] = 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) ck[(int64_t)(tid / 16 + 16 * i) * D + tid % 16] = 0.f;  // slot 0

  // the next chunk's W, Kd and U columns, coalesced, in flight in registers
  float4 pw[NW4], pk[NW4], pu = make_float4(0.f, 0.f, 0.f, 0.f);
  float gn = 0.f;
#pragma unroll
  for (int i = 0; i < NW4; ++i) pw[i] = pk[i] = pu;
#define SPEC_GDN_LOAD(cc)                                                                       \
  {                                                                                             \
    const int64_t it_ = ((int64_t)t * n_chunks + (cc)) * H + h;                                 \
    const float4 *w4_ = reinterpret_cast<const float4 *>(rec_part<D>(ws, it_, RW));             \
    const float4 *k4_ = reinterpret_cast<const float4 *>(rec_part<D>(ws, it_, RKD));            \
    _Pragma("unroll") for (int i = 0; i < NW4; ++i) {                                           \
      pw[i] = w4_[tid + 256 * i];                                                               \
      pk[i] = k4_[tid + 256 * i];                                                               \
    }                                                                                           \
    pu = ld4(rec_part<D>(ws, it_, RU) + (tid / 4) * D + vb * RB + (tid % 4) * 4); /* CT x RB */ \
    gn = gam[it_];                                                                              \
  }
  if (nall > 0) SPEC_GDN_LOAD(0)
  for (int ci = 0; ci < nall; ++ci) {
#pragma unroll
    for (int i = 0; i < NW4; ++i) {
      const int e = (tid + 256 * i) * 4;
      *reinterpret_cast<float4 *>(&Wl[e / D][e % D]) = pw[i];
      *reinterpret_cast<float4 *>(&Kl[e / CT][e % CT]) = pk[i];
    }
    *reinterpret_cast<float4 *>(&Ul[tid / 4][(tid % 4) * 4]) = pu;
    const float gc = gn;
    lds_barrier();
    if (ci + 1 < nall) SPEC_GDN_LOAD(ci + 1)
    // delta = U - W S^T, two accumulation chains over the keys
    f32x4 d0, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) d0[r] = Ul[16 * w + 4 * g + r][c];
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
      const float4 sb = ld4(&Sl[c][g * KW + 4 * i]);
      const float4 wa = ld4(&Wl[16 * w + c][g * KW + 4 * i]);
      d0 = mfma4(-wa.x, sb.x, d0);
      d1 = mfma4(-wa.y, sb.y, d1);
      d0 = mfma4(-wa.z, sb.z, d0);
      d1 = mfma4(-wa.w, sb.w, d1);
    }
    const f32x4 dl = d0 + d1;  // delta[16w + 4g + r][c]
    {
      float *dg = rec_part<D>(ws, ((int64_t)t * n_chunks + ci) * H + h, RDL) +
                  (16 * w + 4 * g) * D + vb * RB + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) dg[r * D] = dl[r];
    }
    if (ci == nfull) break;  // a last partial chunk: no end state (uniform)
    *reinterpret_cast<float4 *>(&DlT[c][16 * w + 4 * g]) = make_float4(dl[0], dl[1], dl[2], dl[3]);
    lds_barrier();
    // S <- gamma S + delta^T Kd
#pragma unroll
    for (int j = 0; j < NT; ++j) S[j] *= gc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 da = ld4(&DlT[c][16 * g + 4 * i]);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float4 kb = ld4(&Kl[16 * (NT * w + j) + c][16 * g + 4 * i]);
        S[j] = mfma4(da.x, kb.x, S[j]);
        S[j] = mfma4(da.y, kb.y, S[j]);
        S[j] = mfma4(da.z, kb.z, S[j]);
        S[j] = mfma4(da.w, kb.w, S[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) Sl[4 * g + r][16 * (NT * w + j) + c] = S[j][r];
    lds_barrier();
    // checkpoint ci + 1, 16 consecutive value rows per key
    float *slot = ck + (int64_t)(ci + 1) * slot_stride;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int key = tid / 16 + 16 * i;
      slot[(int64_t)key * D + tid % 16] = Sl[tid % 16][key];
    }
  }
#undef SPEC_GDN_LOAD
}

// ---------------------------------------------------------------------------
// out: one workgroup of 256 per (tree, chunk, head): o = Q' S_c^T + O' on the
// fp32 matrix cores, as 16 x 16 output tiles (tokens x value rows); wave w takes
// the D/64 adjacent value-row tiles from D/64 w on and all four token tiles of
// each, so a lane's columns of S_c (16 consecutive value rows of one key per
// load, from the key-major checkpoint) are loaded once and used four times. Q'
// comes through LDS.
template <int D>
__global__ __launch_bounds__(256) void gdn_chunk_out_kernel(
    const int32_t *__restrict__ tree_off, const int32_t *__restrict__ tree_trunk_len,
    const float *__restrict__ ws, const float *__restrict__ ckpt, float *__restrict__ out, int H,
    int chunk, int n_chunks, int n_ckpt) {
  constexpr int LD = D + 4, KG = D / 4, NTW = D / 64;  // value-row tiles per wave
  __shared__ __attribute__((aligned(16))) float Ql[CT][LD];
  const int64_t item = blockIdx.x;
  const int h = (int)(item % H);
  const int ch = (int)((item / H) % n_chunks);
  const int t = (int)(item / ((int64_t)H * n_chunks));
  const int T = tree_trunk_len[t];
  const int p0 = ch * chunk;
  if (p0 >= T) return;
  const int L = min(chunk, T - p0);
  const int off = tree_off[t];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, cc = lane & 15;
  {
    const float4 *q4 = reinterpret_cast<const float4 *>(rec_part<D>(ws, item, RQ));
    for (int i = tid; i < CT * D / 4; i += 256) {
      const int e = i * 4;
      *reinterpret_cast<float4 *>(&Ql[e / D][e % D]) = q4[i];
    }
  }
  const float *op = rec_part<D>(ws, item, RO);
  const float *Sc = ckpt + (((int64_t)t * n_ckpt + ch) * H + h) * (int64_t)D * D;
  lds_barrier();
  // the wave's NTW adjacent value-row tiles together, so that the loads of S_c and O'
  // for them cover whole cache lines at once: S_c[16 nt + cc][g KG + i] (key-major, 16
  // lanes read 16 consecutive floats per tile)
  float bv[NTW][KG];
#pragma unroll
  for (int q = 0; q < NTW; ++q)
#pragma unroll
    for (int i = 0; i < KG; ++i) bv[q][i] = Sc[(int64_t)(g * KG + i) * D + 16 * (NTW * w + q) + cc];
#pragma unroll
  for (int mt = 0; mt < CT / 16; ++mt) {
    if (16 * mt >= L) break;  // uniform
    f32x4 acc[NTW];
#pragma unroll
    for (int q = 0; q < NTW; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[q][e] = op[(16 * mt + 4 * g + e) * D + 16 * (NTW * w + q) + cc];
#pragma unroll
    for (int i = 0; i < KG / 4; ++i) {
      const float4 qa = ld4(&Ql[16 * mt + cc][g * KG + 4 * i]);
#pragma unroll
      for (int q = 0; q < NTW; ++q) {
        acc[q] = mfma4(qa.x, bv[q][4 * i], acc[q]);
        acc[q] = mfma4(qa.y, bv[q][4 * i + 1], acc[q]);
        acc[q] = mfma4(qa.z, bv[q][4 * i + 2], acc[q]);
        acc[q] = mfma4(qa.w, bv[q][4 * i + 3], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < NTW; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 16 * mt + 4 * g + e;
        if (s < L) out[((int64_t)(off + p0 + s) * H + h) * D + 16 * (NTW * w + q) + cc] = acc[q][e];
      }
  }
}

// ---------------------------------------------------------------------------
// Branch replay from the trunk pass's cache: one workgroup of 256 per (branch,
// head). Each XCD takes a contiguous run of pairs, head-major with the branches
// in packed (anchor) order, so branches anchored in one chunk follow each other
// on one XCD and read the same checkpoint through its L2. Global operands are
// requested one phase ahead of their use. The branch's m = W - 1 tokens form an MT-row tile
// (features along the ancestry path, A, P, the solve; Q' and O' overwrite q~
// and v~ in LDS), then with 16x16 output tiles on the fp32 matrix cores:
//   Y   = Q' K'^T         (MT x j), scaled by e^{G - g_r}, zero for r >= j, to LDS
//   out = e^{G} Q' S_c^T + O' + Y Delta
// where S_c comes straight from the checkpoint (key-major: a lane's B operand
// is 16 consecutive value rows of one key) and k~, Delta from chunk c's cache.
template <int D, int K, int MT>
__global__ __launch_bounds__(256, MT == 16 ? 3 : 1) void gdn_replay_chunk_kernel(
    const int32_t *__restrict__ tree_off, const int32_t *__restrict__ branch_order,
    const int32_t *__restrict__ branch_tree, const int32_t *__restrict__ branch_anchor,
    const int32_t *__restrict__ branch_len, const int32_t *__restrict__ branch_off,
    const __bf16 *__restrict__ xq, const __bf16 *__restrict__ xk, const __bf16 *__restrict__ xv,
    const float *__restrict__ taps, const float *__restrict__ alpha,
    const float *__restrict__ beta, const float *__restrict__ ckpt, const float *__restrict__ ws,
    const float *__restrict__ glog, float *__restrict__ out, int H, int B, int per_xcd, int chunk,
    int n_chunks, int n_ckpt) {
  constexpr int MTT = MT / 16, NTT = D / 16;  // output tiles along tokens and value rows
  constexpr int PER = MTT * NTT / 4;          // output tiles per wave
  constexpr int KG = D / 4;                   // keys per lane group in a product over keys
  __shared__ __attribute__((aligned(16))) ChunkLds<D, MT> sm;
  __shared__ __attribute__((aligned(16))) float Yl[MT][CT + 4];
  __shared__ float fr[CT];

  const int pair = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (pair >= B * H) return;
  const int h = pair / B, b = branch_order[pair % B];
  const int W = branch_len[b];
  if (W < 2) return;  // the branch has no rows (workgroup-uniform, before any barrier)
  const int m = W - 1;
  const int t = branch_tree[b], a = branch_anchor[b], r0 = branch_off[b];
  const int off = tree_off[t];
  const int c = (a + 1) / chunk, j = a + 1 - c * chunk;  // checkpoint, replayed tokens
  const int tid = threadIdx.x;
  const int64_t citem = ((int64_t)t * n_chunks + c) * H + h;  // chunk c's cache (read when j > 0)
  const float G = j > 0 ? glog[citem * CT + j - 1] : 0.f;
  const float gr = tid < j ? glog[citem * CT + tid] : 0.f;

  // path position p: trunk token p through the anchor, then the branch's rows
  chunk_features<D, K, MT>(sm, [&](int p) { return p <= a ? off + p : r0 + (p - a - 1); }, a + 1, m,
                           xq, xk, xv, taps, alpha, beta, H, h);
  if (tid < CT) fr[tid] = tid < j ? __expf(G - gr) : 0.f;
  chunk_ap<D, MT>(sm);  // its barrier also publishes fr
  {
    const bool isv = tid < D;
    float *dst = isv ? &sm.vf[0][tid] : &sm.qf[0][tid - D];  // O' over v~, Q' over q~
    chunk_solve<D, MT>(sm, [](int, float) {}, [&](int s, float val) { dst[s * (D + 4)] = val; });
  }
  lds_barrier();

  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, cc = lane & 15;
  const float *Sc = ckpt + (((int64_t)t * n_ckpt + c) * H + h) * (int64_t)D * D;
  // the first output tile's column of S_c (key g KG + i, value row 16 nt + cc), in
  // flight during Y
  float bv0[KG];
  {
    const float *sb = Sc + (int64_t)(g * KG) * D + 16 * ((PER * w) / MTT) + cc;
#pragma unroll
    for (int i = 0; i < KG; ++i) bv0[i] = sb[(int64_t)i * D];
  }
  // Y = Q' K'^T over the replayed tokens (tiles of 16 tokens x 16 replayed rows)
  const int nrt = (j + 15) / 16;
  for (int yt = w; yt < MTT * nrt; yt += 4) {
    const int mt = yt % MTT, rt = yt / MTT;
    const float *kr = rec_part<D>(ws, citem, RKF) + (16 * rt + cc) * D + g * KG;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KG / 4; ++i) {
      const float4 qa = ld4(&sm.qf[16 * mt + cc][g * KG + 4 * i]);
      const float4 kb = ld4(kr + 4 * i);
      y = mfma4(qa.x, kb.x, y);
      y = mfma4(qa.y, kb.y, y);
      y = mfma4(qa.z, kb.z, y);
      y = mfma4(qa.w, kb.w, y);
    }
    const float f = fr[16 * rt + cc];
#pragma unroll
    for (int r = 0; r < 4; ++r) Yl[16 * mt + 4 * g + r][16 * rt + cc] = y[r] * f;
  }
  // Q' S_c^T into this wave's output tiles PER w .. PER w + PER - 1 (adjacent value
  // rows, so a wave's loads of S_c and Delta use whole cache lines between them)
  f32x4 acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int ot = PER * w + p, mt = ot % MTT, nt = ot / MTT;
    const float *sb = Sc + (int64_t)(g * KG) * D + 16 * nt + cc;  // key g KG + i, value 16 nt + cc
    acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int i = 0; i < KG / 4; ++i) {
      const float4 qa = ld4(&sm.qf[16 * mt + cc][g * KG + 4 * i]);
      float bb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) bb[e] = p == 0 ? bv0[4 * i + e] : sb[(4 * i + e) * D];
      acc[p] = mfma4(qa.x, bb[0], acc[p]);
      acc[p] = mfma4(qa.y, bb[1], acc[p]);
      acc[p] = mfma4(qa.z, bb[2], acc[p]);
      acc[p] = mfma4(qa.w, bb[3], acc[p]);
    }
  }
  // Delta rows 4 st + g of the first output tile, in flight across the barrier
  float dv0[16];
  if (j > 0) {  // uniform; chunk c's cache exists
    const float *dl = rec_part<D>(ws, citem, RDL) + g * D + 16 * ((PER * w) / MTT) + cc;
#pragma unroll
    for (int st = 0; st < 16; ++st) dv0[st] = dl[(4 * st) * D];
  }
  lds_barrier();  // Y complete
  const float eG = __expf(G);
  const int nsteps = (j + 3) / 4;  // replayed rows r = 4 s + g
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int ot = PER * w + p, mt = ot % MTT, nt = ot / MTT;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[p][r] = eG * acc[p][r] + sm.vf[16 * mt + 4 * g + r][16 * nt + cc];
    if (p == 0) {
#pragma unroll
      for (int st = 0; st < 16; ++st)
        if (st < nsteps) acc[p] = mfma4(Yl[16 * mt + cc][4 * st + g], dv0[st], acc[p]);
    } else if (j > 0) {  // uniform; the tile's 16 Delta loads issued together
      const float *dl = rec_part<D>(ws, citem, RDL) + g * D + 16 * nt + cc;
      float dv[16];
#pragma unroll
      for (int st = 0; st < 16; ++st) dv[st] = dl[(4 * st) * D];
#pragma unroll
      for (int st = 0; st < 16; ++st)
        if (st < nsteps) acc[p] = mfma4(Yl[16 * mt + cc][4 * st + g], dv[st], acc[p]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = 16 * mt + 4 * g + r;
      if (tok < m) out[((int64_t)(r0 + tok) * H + h) * D + 16 * nt + cc] = acc[p][r];
    }
  }
}

template <int D, int K>
hipError_t launch_chunked(const spec_tree_layout &L, int H, int chunk, int n_chunks, int n_ckpt,
                          const void *xq, const void *xk, const void *xv, const float *taps,
                          const float *alpha, const float *beta, float *ckpt, float *out,
                          float *ws, float *gam, float *glog, hipStream_t s) {
  const int64_t items = (int64_t)L.n_trees * n_chunks * H;
  const int64_t pairs = (int64_t)L.n_trees * H;
  hipLaunchKernelGGL((gdn_chunk_prep_kernel<D, K>), dim3((unsigned)items), dim3(256), 0, s,
                     L.tree_off, L.tree_trunk_len, static_cast<const __bf16 *>(xq),
                     static_cast<const __bf16 *>(xk), static_cast<const __bf16 *>(xv), taps, alpha,
                     beta, ws, gam, glog, H, chunk, n_chunks);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  prof_mark(s, "gdn_chunk_prep");
  hipLaunchKernelGGL((gdn_chunk_scan_kernel<D>), dim3((unsigned)((pairs + 7) / 8 * 8 * (D / 16))),
                     dim3(256), 0, s, L.tree_trunk_len, ws, gam, ckpt, H, chunk, n_chunks, n_ckpt,
                     (int)pairs);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  prof_mark(s, "gdn_chunk_scan");
  hipLaunchKernelGGL((gdn_chunk_out_kernel<D>), dim3((unsigned)items), dim3(256), 0, s, L.tree_off,
                     L.tree_trunk_len, ws, ckpt, out, H, chunk, n_chunks, n_ckpt);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  prof_mark(s, "gdn_chunk_out");
  return hipSuccess;
}

template <int D, int K, int MT>
hipError_t launch_replay_chunked(const spec_tree_layout &L, int H, int chunk, int n_chunks,
                                 int n_ckpt, const void *xq, const void *xk, const void *xv,
                                 const float *taps, const float *alpha, const float *beta,
                                 const float *ckpt, const float *ws, const float *glog, float *out,
                                 hipStream_t s) {
  const int64_t pairs = (int64_t)L.n_branches * H;
  if (pairs == 0) return hipSuccess;
  const int64_t per_xcd = (pairs + 7) / 8;
  hipLaunchKernelGGL((gdn_replay_chunk_kernel<D, K, MT>), dim3((unsigned)(per_xcd * 8)), dim3(256), 0,
                     s, L.tree_off, L.branch_order, L.branch_tree, L.branch_anchor, L.branch_len,
                     L.branch_off, static_cast<const __bf16 *>(xq), static_cast<const __bf16 *>(xk),
                     static_cast<const __bf16 *>(xv), taps, alpha, beta, ckpt, ws, glog, out, H,
                     L.n_branches, (int)per_xcd, chunk, n_chunks, n_ckpt);
  return hipGetLastError();
}

struct WorkParts {
  int64_t items;
  size_t rec_floats, glog_off, gam_off, total;  // float offsets; total in bytes
};
WorkParts work_parts(const spec_tree_layout &L, int H, int D, int chunk) {
  WorkParts w;
  const int64_t n_chunks = (L.max_trunk_len + chunk - 1) / chunk;
  w.items = (int64_t)L.n_trees * n_chunks * H;
  w.rec_floats = (size_t)w.items * NREC * CT * D;
  w.glog_off = w.rec_floats;
  w.gam_off = w.glog_off + (size_t)w.items * CT;
  w.total = ((w.gam_off + (size_t)w.items) * sizeof(float) + 255) / 256 * 256;
  return w;
}

}  // namespace

// Workspace of the trunk pass: per (tree, chunk, head) seven CT x D tiles, then
// g [items][CT] and gamma [items]. The token-at-a-time pass (chunk > 64) uses
// none but still asks for a token 256 bytes, so that a NULL workspace always
// means a size query.
size_t gdn_chunk_work_bytes(const spec_tree_layout &L, int H, int D, int chunk) {
  if (chunk > CT) return 256;
  return work_parts(L, H, D, chunk).total;
}

hipError_t launch_gdn_chunked(const spec_tree_layout &L, int H, int D, int K, int chunk, int n_ckpt,
                              const void *xq, const void *xk, const void *xv, const float *taps,
                              const float *alpha, const float *beta, float *ckpt, float *out,
                              void *work, hipStream_t s) {
  const int n_chunks = (L.max_trunk_len + chunk - 1) / chunk;
  const WorkParts wp = work_parts(L, H, D, chunk);
  float *ws = static_cast<float *>(work);
  float *glog = ws + wp.glog_off, *gam = ws + wp.gam_off;
#define SPEC_GDN_CHUNKED(DD, KK)                                                                  \
  if (D == DD && K == KK)                                                                         \
    return launch_chunked<DD, KK>(L, H, chunk, n_chunks, n_ckpt, xq, xk, xv, taps, alpha, beta, \
                                  ckpt, out, ws, gam, glog, s);
  SPEC_GDN_CHUNKED(64, 1) SPEC_GDN_CHUNKED(64, 2) SPEC_GDN_CHUNKED(64, 3) SPEC_GDN_CHUNKED(64, 4)
  SPEC_GDN_CHUNKED(128, 1) SPEC_GDN_CHUNKED(128, 2) SPEC_GDN_CHUNKED(128, 3) SPEC_GDN_CHUNKED(128, 4)
#undef SPEC_GDN_CHUNKED
  return hipErrorInvalidValue;
}

// The branch replay from the cache of the trunk pass (chunk <= 64) that wrote ckpt.
hipError_t launch_gdn_replay_chunked(const spec_tree_layout &L, int H, int D, int K, int chunk,
                                     int n_ckpt, const void *xq, const void *xk, const void *xv,
                                     const float *taps, const float *alpha, const float *beta,
                                     const float *ckpt, const void *work, float *out,
                                     hipStream_t s) {
  const int n_chunks = (L.max_trunk_len + chunk - 1) / chunk;
  const WorkParts wp = work_parts(L, H, D, chunk);
  const float *ws = static_cast<const float *>(work);
  const float *glog = ws + wp.glog_off;
  const int mt = L.max_branch_len - 1 <= 16 ? 16 : L.max_branch_len - 1 <= 32 ? 32 : 64;
#define SPEC_GDN_REPLAY(DD, KK, MM)                                                                 \
  if (D == DD && K == KK && mt == MM)                                                               \
    return launch_replay_chunked<DD, KK, MM>(L, H, chunk, n_chunks, n_ckpt, xq, xk, xv, taps,      \
                                             alpha, beta, ckpt, ws, glog, out, s);
#define SPEC_GDN_REPLAY_K(DD, MM) \
  SPEC_GDN_REPLAY(DD, 1, MM) SPEC_GDN_REPLAY(DD, 2, MM) SPEC_GDN_REPLAY(DD, 3, MM) SPEC_GDN_REPLAY(DD, 4, MM)
  SPEC_GDN_REPLAY_K(64, 16) SPEC_GDN_REPLAY_K(64, 32) SPEC_GDN_REPLAY_K(64, 64)
  SPEC_GDN_REPLAY_K(128, 16) SPEC_GDN_REPLAY_K(128, 32) SPEC_GDN_REPLAY_K(128, 64)
#undef SPEC_GDN_REPLAY_K
#undef SPEC_GDN_REPLAY
  return hipErrorInvalidValue;
}

}  // namespace spec
