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
//   scan (tree, head, 16 value rows): S <- gamma S + (U - W S^T)^T Kd over the
//        full chunks in order on the fp32 matrix cores, storing each end state
//        as the next checkpoint.
//   out  (tree, chunk, head): o = Q' S_c^T + O' from checkpoint c.
// A chunk tile always has 64 rows; rows past the chunk's tokens are zero.
// Intermediates live in a caller-provided workspace.
#include "common.h"
#include "gdn_util.h"

namespace spec {

namespace {

using gdn::silu_f;
using gdn::wave_sum;

constexpr int CT = 64;    // rows of a chunk tile (the chunk length is at most this)
constexpr int NREC = 5;   // per (tree, chunk, head): W, U, Kd, Q', O', each CT x D
enum { RW = 0, RU = 1, RKD = 2, RQ = 3, RO = 4 };

__device__ inline float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

template <int D>
__device__ inline float *rec_part(float *ws, int64_t item, int part) {
  return ws + (item * NREC + part) * (int64_t)(CT * D);
}
template <int D>
__device__ inline const float *rec_part(const float *ws, int64_t item, int part) {
  return ws + (item * NREC + part) * (int64_t)(CT * D);
}

// ---------------------------------------------------------------------------
// prep: one workgroup of 256 per (tree, chunk, head), item = (t * n_chunks + c) * H + h.
template <int D, int K>
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(
    const int32_t *__restrict__ tree_off, const int32_t *__restrict__ tree_trunk_len,
    const __bf16 *__restrict__ xq, const __bf16 *__restrict__ xk, const __bf16 *__restrict__ xv,
    const float *__restrict__ taps, const float *__restrict__ alpha,
    const float *__restrict__ beta, float *__restrict__ ws, float *__restrict__ gam, int H,
    int chunk, int n_chunks) {
  constexpr int LD = D + 4;  // padded rows: 16 consecutive rows start 4 banks apart
  __shared__ __attribute__((aligned(16))) float kf[CT][LD];
  __shared__ __attribute__((aligned(16))) float qf[CT][LD];
  __shared__ __attribute__((aligned(16))) float vf[CT][D];
  __shared__ __attribute__((aligned(16))) float Al[CT][CT + 4];
  __shared__ __attribute__((aligned(16))) float Pl[CT][CT + 4];
  __shared__ float g[CT], eg[CT], bt[CT], nk[CT], nq[CT];

  const int64_t item = blockIdx.x;
  const int h = (int)(item % H);
  const int c = (int)((item / H) % n_chunks);
  const int t = (int)(item / ((int64_t)H * n_chunks));
  const int T = tree_trunk_len[t];
  const int p0 = c * chunk;  // trunk position of the tile's row 0
  if (p0 >= T) return;       // workgroup-uniform, before any barrier
  const int L = min(chunk, T - p0);
  const int off = tree_off[t];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // features before the norms: the convolution along the trunk, then SiLU.
  // Thread (d, group) takes channel d of CT / G consecutive tokens; the raw
  // rows they read (K - 1 more before the first) are all loaded up front.
  {
    constexpr int G = 256 / D, TPG = CT / G, NR = TPG + K - 1;
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
    for (int i = 0; i < NR; ++i) {  // raw row i is trunk position p0 + s0 - (K - 1) + i
      const int p = p0 + s0 - (K - 1) + i;
      const bool ok = p >= 0 && p < p0 + L;
      const int64_t at = ((int64_t)(off + (ok ? p : 0)) * H + h) * D + d;
      const float q = (float)xq[at], k = (float)xk[at], v = (float)xv[at];
      rq[i] = ok ? q : 0.f;
      rk[i] = ok ? k : 0.f;
      rv[i] = ok ? v : 0.f;
    }
#pragma unroll
    for (int s = 0; s < TPG; ++s) {
      float aq = 0.f, ak = 0.f, av = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) {  // tap j reads position p0 + s0 + s - j
        aq = fmaf(tq[j], rq[s + K - 1 - j], aq);
        ak = fmaf(tk[j], rk[s + K - 1 - j], ak);
        av = fmaf(tv[j], rv[s + K - 1 - j], av);
      }
      const bool live = s0 + s < L;
      qf[s0 + s][d] = live ? silu_f(aq) : 0.f;
      kf[s0 + s][d] = live ? silu_f(ak) : 0.f;
      vf[s0 + s][d] = live ? silu_f(av) : 0.f;
    }
  }
  // gates: running sum of log alpha (a wave scan); rows past L have alpha = 1, beta = 0
  if (wv == 0) {
    float la = 0.f, b = 0.f;
    if (lane < L) {
      const int64_t gi = (int64_t)(off + p0 + lane) * H + h;
      la = __logf(alpha[gi]);
      b = beta[gi];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(la, o);
      if (lane >= o) la += y;
    }
    g[lane] = la;
    eg[lane] = __expf(la);
    bt[lane] = b;
  }
  __syncthreads();
  // L2 norms of k and q per token (wave wv takes tokens wv, wv + 4, ...)
  const float qscale = 1.f / sqrtf((float)D);
  for (int s = wv; s < CT; s += 4) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int d = lane; d < D; d += 64) {
      sk = fmaf(kf[s][d], kf[s][d], sk);
      sq = fmaf(qf[s][d], qf[s][d], sq);
    }
    sk = wave_sum(sk);
    sq = wave_sum(sq);
    if (lane == 0) {
      nk[s] = s < L ? __builtin_amdgcn_rsqf(sk) : 0.f;
      nq[s] = s < L ? qscale * __builtin_amdgcn_rsqf(sq) : 0.f;
    }
  }
  __syncthreads();
  for (int i = tid; i < CT * D; i += 256) {
    const int s = i / D, d = i % D;
    kf[s][d] *= nk[s];
    qf[s][d] *= nq[s];
  }
  __syncthreads();

  // A_sr (r < s) and P_sr (r <= s): lane r holds k_r in 32-column pieces, wave
  // wv takes rows s = 16 wv .. 16 wv + 15, whose k_s and q_s are LDS broadcasts.
  {
    const int r = lane;
    float accA[16], accP[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) accA[i] = accP[i] = 0.f;
#pragma unroll 1
    for (int d0 = 0; d0 < D; d0 += 32) {
      float kr[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 x = ld4(&kf[r][d0 + 4 * i]);
        kr[4 * i] = x.x;
        kr[4 * i + 1] = x.y;
        kr[4 * i + 2] = x.z;
        kr[4 * i + 3] = x.w;
      }
#pragma unroll
      for (int si = 0; si < 16; ++si) {
        const int s = 16 * wv + si;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 ks = ld4(&kf[s][d0 + 4 * i]);
          const float4 qs = ld4(&qf[s][d0 + 4 * i]);
          accA[si] = fmaf(ks.x, kr[4 * i], accA[si]);
          accA[si] = fmaf(ks.y, kr[4 * i + 1], accA[si]);
          accA[si] = fmaf(ks.z, kr[4 * i + 2], accA[si]);
          accA[si] = fmaf(ks.w, kr[4 * i + 3], accA[si]);
          accP[si] = fmaf(qs.x, kr[4 * i], accP[si]);
          accP[si] = fmaf(qs.y, kr[4 * i + 1], accP[si]);
          accP[si] = fmaf(qs.z, kr[4 * i + 2], accP[si]);
          accP[si] = fmaf(qs.w, kr[4 * i + 3], accP[si]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the broadcast reads near their FMAs
      }
    }
#pragma unroll
    for (int si = 0; si < 16; ++si) {
      const int s = 16 * wv + si;
      const float e = __expf(g[s] - g[r]);  // used only where r <= s, so e <= 1
      Al[s][r] = r < s ? e * accA[si] : 0.f;
      Pl[s][r] = r <= s ? e * accP[si] : 0.f;
    }
  }
  __syncthreads();

  // The triangular solve and P X, one column j of X = [U | W] per thread, in
  // registers; rows of A and P are LDS broadcasts.
  const int j = tid;
  if (j < 2 * D) {
    // column j of the right-hand side: v (j < D) or e^g k; branch-free so the
    // whole solve stays one scheduling region
    const bool isv = j < D;
    const float *rhs = isv ? &vf[0][j] : &kf[0][j - D];
    const int rstride = isv ? D : LD;
    const float *qcol = &qf[0][isv ? 0 : j - D];
    float x[CT];
#pragma unroll
    for (int s = 0; s < CT; ++s) x[s] = 0.f;
#pragma unroll
    for (int s = 0; s < CT; ++s) {
      float acc = rhs[s * rstride] * (isv ? 1.f : eg[s]);
#pragma unroll
      for (int r0 = 0; r0 < s; r0 += 4) {  // A_sr = 0 and x_r = 0 for r >= s
        const float4 a = ld4(&Al[s][r0]);
        acc = fmaf(-a.x, x[r0], acc);
        acc = fmaf(-a.y, x[r0 + 1], acc);
        acc = fmaf(-a.z, x[r0 + 2], acc);
        acc = fmaf(-a.w, x[r0 + 3], acc);
      }
      x[s] = bt[s] * acc;
    }
    float *dst_x = isv ? rec_part<D>(ws, item, RU) + j : rec_part<D>(ws, item, RW) + (j - D);
#pragma unroll
    for (int s = 0; s < CT; ++s) dst_x[s * D] = x[s];
    float *dst_y = isv ? rec_part<D>(ws, item, RO) + j : rec_part<D>(ws, item, RQ) + (j - D);
#pragma unroll
    for (int s = 0; s < CT; ++s) {
      float acc = 0.f;
#pragma unroll
      for (int r0 = 0; r0 <= s; r0 += 4) {  // P_sr = 0 for r > s
        const float4 p = ld4(&Pl[s][r0]);
        acc = fmaf(p.x, x[r0], acc);
        acc = fmaf(p.y, x[r0 + 1], acc);
        acc = fmaf(p.z, x[r0 + 2], acc);
        acc = fmaf(p.w, x[r0 + 3], acc);
      }
      const float qv = qcol[s * LD];
      dst_y[s * D] = isv ? acc : eg[s] * qv - acc;  // O' = P U; Q' = e^g Q - P W
    }
  }
  // Kd_s = e^{g_{L-1} - g_s} k_s (g is flat past L, so g[CT-1] = g[L-1]),
  // stored transposed: key-major, CT tokens per key
  {
    float *kd = rec_part<D>(ws, item, RKD);
    const float gl = g[CT - 1];
    for (int i = tid; i < CT * D; i += 256) {
      const int key = i / CT, s = i % CT;
      kd[i] = __expf(gl - g[s]) * kf[s][key];
    }
  }
  if (tid == 0) gam[item] = eg[CT - 1];
}

// ---------------------------------------------------------------------------
// scan: one workgroup of 256 per (tree, head, 16 value rows), on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds C[4 (l / 16) + r][l % 16], r = 0..3). Per chunk:
//   delta (64 tokens x 16 rows) = U - W S^T: wave w takes tokens 16w..16w+15,
//        K runs over the keys, lane group g taking keys g D/4 .. (g+1) D/4 - 1;
//   S (16 rows x D keys) = gamma S + delta^T Kd: wave w owns D/64 tiles of 16
//        keys in registers, K runs over the tokens, group g taking 16g .. 16g+15.
// W, Kd (stored key-major) and U reach registers straight from the workspace
// one chunk ahead; delta and S pass between waves through LDS. The D / 16 row
// blocks of one (tree, head) take workgroup ids 8 apart, so they run on one
// XCD and share its L2 for W and Kd.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void gdn_chunk_scan_kernel(
    const int32_t *__restrict__ tree_trunk_len, const float *__restrict__ ws,
    const float *__restrict__ gam, float *__restrict__ ckpt, int H, int chunk, int n_chunks,
    int n_ckpt, int n_pairs) {
  constexpr int RB = 16, NB = D / RB;
  constexpr int KW = D / 4;   // keys per lane group in the delta product
  constexpr int NT = D / 64;  // 16-key state tiles per wave
  __shared__ __attribute__((aligned(16))) float Sl[RB][D + 4];    // S of the block
  __shared__ __attribute__((aligned(16))) float DlT[RB][CT + 4];  // delta, row-major by value row

  const int x8 = blockIdx.x % 8, y8 = blockIdx.x / 8;
  const int vb = y8 % NB, pair = x8 + 8 * (y8 / NB);
  if (pair >= n_pairs) return;
  const int h = pair % H, t = pair / H;
  const int nfull = tree_trunk_len[t] / chunk;  // chunks whose end state is a checkpoint
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

  // one chunk's operands for this lane:
  //   W[16w + c][g KW ..], KdT[16 (NT w + j) + c][16 g ..], U[16w + 4g + r][vb RB + c], gamma
  float4 wn[KW / 4], kn[NT][4];
  float un[4], gn = 0.f;
#pragma unroll
  for (int i = 0; i < KW / 4; ++i) wn[i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) kn[j][i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int r = 0; r < 4; ++r) un[r] = 0.f;
#define SPEC_GDN_LOAD(cc)                                                                  \
  {                                                                                        \
    const int64_t it_ = ((int64_t)t * n_chunks + (cc)) * H + h;                            \
    const float *W_ = rec_part<D>(ws, it_, RW) + (16 * w + c) * D + g * KW;                \
    const float *K_ = rec_part<D>(ws, it_, RKD) + 16 * g;                                  \
    const float *U_ = rec_part<D>(ws, it_, RU) + (16 * w + 4 * g) * D + vb * RB + c;       \
    _Pragma("unroll") for (int i = 0; i < KW / 4; ++i) wn[i] = ld4(W_ + 4 * i);            \
    _Pragma("unroll") for (int j = 0; j < NT; ++j)                                         \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                        \
        kn[j][i] = ld4(K_ + (16 * (NT * w + j) + c) * CT + 4 * i);                          \
    _Pragma("unroll") for (int r = 0; r < 4; ++r) un[r] = U_[r * D];                       \
    gn = gam[it_];                                                                         \
  }
  if (nfull > 0) SPEC_GDN_LOAD(0)
  for (int ci = 0; ci < nfull; ++ci) {
    float4 wc[KW / 4], kc[NT][4];
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) wc[i] = wn[i];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) kc[j][i] = kn[j][i];
    f32x4 d0 = {un[0], un[1], un[2], un[3]}, d1 = {0.f, 0.f, 0.f, 0.f};
    const float gc = gn;
    if (ci + 1 < nfull) SPEC_GDN_LOAD(ci + 1)
    // delta = U - W S^T, two accumulation chains over the keys
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
      const float4 sb = ld4(&Sl[c][g * KW + 4 * i]);
      d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(-wc[i].x, sb.x, d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(-wc[i].y, sb.y, d1, 0, 0, 0);
      d0 = __builtin_amdgcn_mfma_f32_16x16x4f32(-wc[i].z, sb.z, d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x4f32(-wc[i].w, sb.w, d1, 0, 0, 0);
    }
    const f32x4 dl = d0 + d1;  // delta[16w + 4g + r][c]
    *reinterpret_cast<float4 *>(&DlT[c][16 * w + 4 * g]) = make_float4(dl[0], dl[1], dl[2], dl[3]);
    __syncthreads();
    // S <- gamma S + delta^T Kd
#pragma unroll
    for (int j = 0; j < NT; ++j) S[j] *= gc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 da = ld4(&DlT[c][16 * g + 4 * i]);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(da.x, kc[j][i].x, S[j], 0, 0, 0);
        S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(da.y, kc[j][i].y, S[j], 0, 0, 0);
        S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(da.z, kc[j][i].z, S[j], 0, 0, 0);
        S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(da.w, kc[j][i].w, S[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) Sl[4 * g + r][16 * (NT * w + j) + c] = S[j][r];
    __syncthreads();
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
// out: one workgroup of 256 per (tree, chunk, head): o = Q' S_c^T + O'.
template <int D>
__global__ __launch_bounds__(256) void gdn_chunk_out_kernel(
    const int32_t *__restrict__ tree_off, const int32_t *__restrict__ tree_trunk_len,
    const float *__restrict__ ws, const float *__restrict__ ckpt, float *__restrict__ out, int H,
    int chunk, int n_chunks, int n_ckpt) {
  constexpr int LD = D + 4, G = 256 / D, RPT = CT / G;
  __shared__ __attribute__((aligned(16))) float Ql[CT][LD];
  const int64_t item = blockIdx.x;
  const int h = (int)(item % H);
  const int c = (int)((item / H) % n_chunks);
  const int t = (int)(item / ((int64_t)H * n_chunks));
  const int T = tree_trunk_len[t];
  const int p0 = c * chunk;
  if (p0 >= T) return;
  const int L = min(chunk, T - p0);
  const int off = tree_off[t];
  const int tid = threadIdx.x;
  {
    const float4 *q4 = reinterpret_cast<const float4 *>(rec_part<D>(ws, item, RQ));
    for (int i = tid; i < CT * D / 4; i += 256) {
      const int e = i * 4;
      *reinterpret_cast<float4 *>(&Ql[e / D][e % D]) = q4[i];
    }
  }
  const int v = tid % D, sg = tid / D;  // sg is uniform across a wave
  const float *op = rec_part<D>(ws, item, RO);
  float acc[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) acc[i] = op[(sg + G * i) * D + v];
  __syncthreads();
  const float *sc = ckpt + (((int64_t)t * n_ckpt + c) * H + h) * (int64_t)D * D + v;
#pragma unroll 1
  for (int k0 = 0; k0 < D; k0 += 32) {
    float sr[32];
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) sr[kk] = sc[(int64_t)(k0 + kk) * D];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int s = sg + G * i;
#pragma unroll
      for (int kk = 0; kk < 32; kk += 4) {
        const float4 q4 = ld4(&Ql[s][k0 + kk]);
        acc[i] = fmaf(q4.x, sr[kk], acc[i]);
        acc[i] = fmaf(q4.y, sr[kk + 1], acc[i]);
        acc[i] = fmaf(q4.z, sr[kk + 2], acc[i]);
        acc[i] = fmaf(q4.w, sr[kk + 3], acc[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int s = sg + G * i;
    if (s < L) out[((int64_t)(off + p0 + s) * H + h) * D + v] = acc[i];
  }
}

template <int D, int K>
hipError_t launch_chunked(const spec_tree_layout &L, int H, int chunk, int n_chunks, int n_ckpt,
                          const void *xq, const void *xk, const void *xv, const float *taps,
                          const float *alpha, const float *beta, float *ckpt, float *out,
                          float *ws, float *gam, hipStream_t s) {
  const int64_t items = (int64_t)L.n_trees * n_chunks * H;
  const int64_t pairs = (int64_t)L.n_trees * H;
  hipLaunchKernelGGL((gdn_chunk_prep_kernel<D, K>), dim3((unsigned)items), dim3(256), 0, s,
                     L.tree_off, L.tree_trunk_len, static_cast<const __bf16 *>(xq),
                     static_cast<const __bf16 *>(xk), static_cast<const __bf16 *>(xv), taps, alpha,
                     beta, ws, gam, H, chunk, n_chunks);
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

}  // namespace

// Workspace of the trunk pass; the token-at-a-time pass (chunk > 64) uses none
// but still asks for a token 256 bytes, so that a NULL workspace always means a
// size query.
size_t gdn_chunk_work_bytes(const spec_tree_layout &L, int H, int D, int chunk) {
  if (chunk > CT) return 256;
  const int64_t n_chunks = (L.max_trunk_len + chunk - 1) / chunk;
  const int64_t items = (int64_t)L.n_trees * n_chunks * H;
  const size_t rec = (size_t)items * NREC * CT * D * sizeof(float);
  return rec + ((size_t)items * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_gdn_chunked(const spec_tree_layout &L, int H, int D, int K, int chunk, int n_ckpt,
                              const void *xq, const void *xk, const void *xv, const float *taps,
                              const float *alpha, const float *beta, float *ckpt, float *out,
                              void *work, hipStream_t s) {
  const int n_chunks = (L.max_trunk_len + chunk - 1) / chunk;
  const int64_t items = (int64_t)L.n_trees * n_chunks * H;
  float *ws = static_cast<float *>(work);
  float *gam = ws + items * NREC * CT * D;
#define SPEC_GDN_CHUNKED(DD, KK)                                                                  \
  if (D == DD && K == KK)                                                                         \
    return launch_chunked<DD, KK>(L, H, chunk, n_chunks, n_ckpt, xq, xk, xv, taps, alpha, beta, \
                                  ckpt, out, ws, gam, s);
  SPEC_GDN_CHUNKED(64, 1) SPEC_GDN_CHUNKED(64, 2) SPEC_GDN_CHUNKED(64, 3) SPEC_GDN_CHUNKED(64, 4)
  SPEC_GDN_CHUNKED(128, 1) SPEC_GDN_CHUNKED(128, 2) SPEC_GDN_CHUNKED(128, 3) SPEC_GDN_CHUNKED(128, 4)
#undef SPEC_GDN_CHUNKED
  return hipErrorInvalidValue;
}

}  // namespace spec
