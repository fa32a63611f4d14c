// E2E-TV surrogate, loss and gradient with respect to the draft logits.
//
// [SpecOPD notes page, "Equations"]: alpha_{b,i} = sum_v min(q_v, p_v) over the
// full vocabulary; L = 1 - (1/(BW)) sum_b sum_j prod_{i<=j} alpha_{b,i}; samples
// and the teacher are fixed when differentiating; teacher mass outside the draft
// support is kept. [SpecOPD notes page, "Inputs and code mapping"]: low
// precision is promoted to float32; NaN draft entries are inactive support.
//
// Main path (bf16 rows whose length is a multiple of 8, every branch spanning
// at most two steps of the team pipeline): one cooperative kernel,
// e2etv_fused_team_kernel, reads each logit once and writes each gradient
// element once (8 bytes per element). Teams of workgroups split every row by
// vocabulary slices, exchange per-member log-sum-exps and (alpha, S) partials
// through agent-scope atomics, form each row's coefficient
// c_s = dL/d alpha_s = -w A_{i-1} G_i from its branch's alphas, and write
// grad[s,u] = c_s q_u (1[z'_u < y'_u] - S_s) from the row slice still held in
// registers (z' = z log2(e) - lse2(z) is log2 q, y' likewise log2 p).
// e2etv_loss_kernel then adds the per-branch sums of prefix products in
// branch order. Details above the kernel.
//
// Fallback path (float32 rows, other lengths, long branches), three kernels:
//   statistics   e2etv_stats_team_kernel (single read of each row by a team) or
//                e2etv_stats_kernel (one workgroup per row, two passes): the
//                log-sum-exps, alpha = sum 2^min(z', y'), S = sum over {z' < y'}
//                of 2^z', and the decision z' < y' as a bitmask;
//   e2etv_scan   one wave per branch: suffix sums G and prefix products A give
//                c_s (no division); the loss is reduced in float64 in a fixed order;
//   e2etv_grad   grad[s,u] from the draft row and the bitmask, written once.
// Every reduction has a fixed order, so results are bitwise reproducible. The
// strict test z' < y' is the same expression wherever {q < p} is used, so the
// set used for S and for the gradient is the same set.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace spec {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStatThreads = 1024;
constexpr int kGradThreads = 256;
constexpr int kGradVecs = 4;  // 8-element vectors per thread in the gradient kernel

__device__ inline float sanitize(float z) { return __builtin_isnan(z) ? -INFINITY : z; }

__device__ inline void load8(const __bf16 *p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ inline void load8(const float *p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ inline float load1(const __bf16 *p) { return (float)*p; }
__device__ inline float load1(const float *p) { return *p; }

// (max, sum of 2^((x - max) log2 e)) merge; an empty side has max = -inf, sum = 0.
__device__ inline void lse_merge(float &m, float &s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
  m = mn;
}

__device__ inline void lse_add_chunk(float &m, float &s, const float (&x)[8]) {
  float cm = x[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) cm = fmaxf(cm, x[k]);
  if (cm > m) {
    s = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - cm) * kLog2e);
    m = cm;
  }
  if (m == -INFINITY) return;
  const float nm = -m * kLog2e;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += __builtin_amdgcn_exp2f(fmaf(x[k], kLog2e, nm));
}

template <int NT>
__device__ inline void block_lse(float &m, float &s, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    lse_merge(m, s, m2, s2);
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[2 * w] = m;
    red[2 * w + 1] = s;
  }
  __syncthreads();
  m = red[0];
  s = red[1];
  for (int k = 1; k < NT / 64; ++k) lse_merge(m, s, red[2 * k], red[2 * k + 1]);
}

template <int NT>
__device__ inline float block_sum(float x, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float t = red[0];
  for (int k = 1; k < NT / 64; ++k) t += red[k];
  return t;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kStatThreads) void e2etv_stats_kernel(
    const T *__restrict__ draft, const T *__restrict__ teacher, int64_t n_rows, int64_t V,
    float2 *__restrict__ part, float *__restrict__ lse_q2,
    float *__restrict__ lse_p2, uint8_t *__restrict__ bits, int64_t bits_row,
    unsigned *__restrict__ ticket) {
  __shared__ float red[2 * kStatThreads / 64];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid == 0) *ticket = 0u;  // the scan kernel's ticket
  for (int64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
  const T *z = draft + row * V;
  const T *y = teacher + row * V;

  float mz = -INFINITY, sz = 0.f, my = -INFINITY, sy = 0.f;
  if (VEC) {
    for (int64_t i = (int64_t)tid * 8; i < V; i += kStatThreads * 8) {
      float a[8], b[8];
      load8(z + i, a);
      load8(y + i, b);
#pragma unroll
      for (int k = 0; k < 8; ++k) a[k] = sanitize(a[k]);
      lse_add_chunk(mz, sz, a);
      lse_add_chunk(my, sy, b);
    }
  } else {
    for (int64_t i = tid; i < V; i += kStatThreads) {
      const float a = sanitize(load1(z + i)), b = load1(y + i);
      lse_merge(mz, sz, a, a == -INFINITY ? 0.f : 1.f);
      lse_merge(my, sy, b, 1.f);
    }
  }
  block_lse<kStatThreads>(mz, sz, red);
  block_lse<kStatThreads>(my, sy, red);
  const float lz2 = mz * kLog2e + log2f(sz);  // log2 of sum_v 2^(z_v log2 e)
  const float ly2 = my * kLog2e + log2f(sy);

  float al = 0.f, ss = 0.f;
  if (VEC) {
    uint8_t *brow = bits + row * bits_row;
    for (int64_t i = (int64_t)tid * 8; i < V; i += kStatThreads * 8) {
      float a[8], b[8];
      load8(z + i, a);
      load8(y + i, b);
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float za = fmaf(sanitize(a[k]), kLog2e, -lz2);  // log2 q
        const float yb = fmaf(b[k], kLog2e, -ly2);            // log2 p
        const float e = __builtin_amdgcn_exp2f(fminf(za, yb));
        const bool in = za < yb;
        al += e;
        ss += in ? e : 0.f;
        m |= (uint32_t)in << k;
      }
      brow[i / 8] = (uint8_t)m;  // the gradient reads this decision instead of the teacher row
    }
  } else {
    for (int64_t i = tid; i < V; i += kStatThreads) {
      const float za = fmaf(sanitize(load1(z + i)), kLog2e, -lz2);
      const float yb = fmaf(load1(y + i), kLog2e, -ly2);
      const float e = __builtin_amdgcn_exp2f(fminf(za, yb));
      al += e;
      ss += za < yb ? e : 0.f;
    }
  }
  al = block_sum<kStatThreads>(al, red);
  ss = block_sum<kStatThreads>(ss, red);
  if (tid == 0) {
    part[row] = make_float2(al, ss);
    lse_q2[row] = lz2;
    lse_p2[row] = ly2;
  }
  }
}

// ---------------------------------------------------------------------------
// Single-read statistics for bf16 rows whose length is a multiple of 8.
//
// A cooperative grid is cut into teams of T workgroups (one per CU); team t
// takes rows t, t + n_teams, ... and member j owns vector slice j of every
// row, so every logit is read from HBM once. Each row goes through
//   pass 1   (data waves) log2-sum-exp2 of z log2(e) and of y log2(e) per wave;
//   exchange (sync wave) the wave values merge into the member's, which goes into
//            the row's slot for this member; the other members' slots of the row
//            are polled and merged in member order: lse2(z), lse2(y);
//   pass 2   (data waves) alpha and S over the slice, and the indicator bits;
// and the member's alpha and S go to part[row][j], which the scan kernel adds up
// in member order. The work is a three-stage pipeline over three register
// buffers: in step i the data waves run pass 1 of row i, then pass 2 of row
// i - 1, then issue the loads of row i + 2 into the buffer row i - 1 has freed,
// while the sync wave runs the exchange of row i. One workgroup barrier per
// step separates them, so the exchange is hidden behind a pass of compute.
//
// The exchange runs in a wave of its own so that its loads never queue behind
// the data waves' loads (a wave's loads complete in issue order). Slots are
// 64-bit words, (lse2 z, lse2 y), written once per row by one atomic store and
// cleared to all-ones before the launch; the all-ones pattern is no value a
// member writes (NaNs are stored canonical). Agent-scope atomic loads and stores
// reach the coherence point, so they are seen across XCDs, whose L2s are not
// coherent with each other, without an L2 writeback or invalidate. The poll is
// bounded: on a timeout the status word is raised, every member leaves, and the
// scan kernel turns alpha and the loss into NaN.
//
// Every merge (lanes within a wave, waves within a member, members within a row)
// is a fixed reduction tree, so results are bitwise reproducible.

constexpr int kTeamThreads = 1024;
constexpr int kTeamData = kTeamThreads - 64;  // 15 data waves; the last wave runs the exchange
constexpr int kTeamDataWaves = kTeamData / 64;
constexpr unsigned kTeamSpinLimit = 1u << 20;
constexpr uint32_t kNegInf2 = 0xff80ff80u;    // two bf16 -inf
constexpr unsigned long long kSlotEmpty = ~0ull;

struct TeamArgs {
  const __bf16 *z, *y;
  int64_t R, V8;                // rows, 8-element vectors per row
  int32_t T, n_teams;
  float *lse_q2, *lse_p2;
  float2 *part;                 // [R][T] (alpha, S) member partials
  uint8_t *bits;
  int64_t bits_row;
  unsigned long long *xchg;     // [R][T] member (lse2 z, lse2 y) slots, all-ones until written
  unsigned *status;
};

__device__ inline float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Two more spellings of the bf16 -> f32 unpack, so that the compiler cannot keep
// one pass's unpacked values alive for a later one (that would double the
// registers a slice needs). v_perm_b32 picks bytes of {src0, src1}: 0-3 from
// src1, 4-7 from src0, 0x0c gives a zero byte.
__device__ inline float lo_p(uint32_t w) { return __uint_as_float(__builtin_amdgcn_perm(0u, w, 0x01000c0cu)); }
__device__ inline float hi_p(uint32_t w) { return __uint_as_float(__builtin_amdgcn_perm(0u, w, 0x03020c0cu)); }
__device__ inline float lo_q(uint32_t w) { return __uint_as_float(__builtin_amdgcn_perm(w, 0u, 0x05040c0cu)); }
__device__ inline float hi_q(uint32_t w) { return __uint_as_float(__builtin_amdgcn_perm(w, 0u, 0x07060c0cu)); }
__device__ inline uint32_t word(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Wave reductions in registers: DPP within rows of 16 lanes (xor 1, xor 2, then
// the half-row and row mirrors), then the lane swaps across rows (l ^ 16, l ^ 32).
// Every step combines a lane with its partner by a commutative operation, so
// every lane ends with the same bits.
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ inline float dpp_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float dpp_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum over each row of 16 lanes (the first four steps of dpp_sum); every lane
// of a row ends with the same bits.
__device__ inline float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
constexpr int kTeamRows = kTeamDataWaves * 4;  // 16-lane rows of the data waves

// log2 sum_lanes 2^l over a wave (l = -inf: no contribution).
__device__ inline float wave_lse2(float l) {
  const float M = dpp_max(l);
  if (M == -INFINITY) return -INFINITY;
  return M + log2f(dpp_sum(__builtin_amdgcn_exp2f(l - M)));
}
// Two bf16 in one word with NaN halves replaced by -inf (inactive draft support).
__device__ inline uint32_t nan_to_neginf2(uint32_t w) {
  if ((w & 0x7fffu) > 0x7f80u) w = (w & 0xffff0000u) | 0xff80u;
  if (((w >> 16) & 0x7fffu) > 0x7f80u) w = (w & 0x0000ffffu) | 0xff800000u;
  return w;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// A row slice of one thread: VPL vectors of the draft and of the teacher.
template <int VPL>
struct Slice {
  uint4 z[VPL], y[VPL];
};

// Issue the loads of this thread's vectors of row r (vector k at slice offset
// tid + kTeamData k); nothing waits for the data here. Reads past the row end
// return zero and are masked before use. With `valid` false the range is empty:
// the loads are issued (so every path issues the same memory operations, which
// keeps the compiler's wait counts exact) but read nothing.
template <int VPL>
__device__ inline void team_load(Slice<VPL> &b, const TeamArgs &a, int64_t r, uint32_t voff, bool valid) {
  const uint32_t bytes = valid ? (uint32_t)(a.V8 * 16) : 0u;
  r = valid ? r : 0;
  const __amdgpu_buffer_rsrc_t rz = row_rsrc(a.z + r * a.V8 * 8, bytes);
  const __amdgpu_buffer_rsrc_t ry = row_rsrc(a.y + r * a.V8 * 8, bytes);
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rz, voff, k * kTeamData * 16, 0);
    b.z[k] = make_uint4(u.x, u.y, u.z, u.w);
  }
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(ry, voff, k * kTeamData * 16, 0);
    b.y[k] = make_uint4(u.x, u.y, u.z, u.w);
  }
}

// sum 2^(x log2 e + nm) over this thread's vectors.
template <int VPL>
__device__ inline float sum_shifted(const uint4 (&v)[VPL], float nm) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = word(v[k], i);
      s += __builtin_amdgcn_exp2f(fmaf(lo_p(w), kLog2e, nm));
      s += __builtin_amdgcn_exp2f(fmaf(hi_p(w), kLog2e, nm));
    }
  return s;
}

// log2 sum 2^(x log2 e) of one array over each 16-lane row of the wave, each
// element taken as 2^(x log2 e - c) with a wave-uniform shift c (log2 units).
// c comes from the caller (an earlier row's log-sum-exp) or, if it is -inf,
// from the wave max of a sample (every lane's first vector). If any row's sum
// then leaves [2^-60, 2^64) - too far from the row's own scale for full
// precision, an overflow, or a NaN (a NaN draft entry) - the wave takes the
// exact wave max as the shift instead, after NaN draft entries become -inf in
// the words themselves (pass 2 then sees them as -inf too).
template <int VPL>
__device__ inline float rows_lse2_of(uint4 (&v)[VPL], bool draft, float c) {
  if (c == -INFINITY) {  // wave-uniform
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = word(v[0], i);
      m = __builtin_fmaxf(__builtin_fmaxf(m, lo_f(w)), hi_f(w));
    }
    c = dpp_max(m) * kLog2e;
  }
  float s = 0.f;
  if (c > -INFINITY && c < INFINITY) s = row16_sum(sum_shifted<VPL>(v, -c));
  if (__any(!(s >= 0x1p-60f && s < 0x1p64f))) {  // wave-uniform
    if (draft) {
#pragma unroll
      for (int k = 0; k < VPL; ++k)
        v[k] = make_uint4(nan_to_neginf2(v[k].x), nan_to_neginf2(v[k].y), nan_to_neginf2(v[k].z),
                          nan_to_neginf2(v[k].w));
    }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = word(v[k], i);
        m = __builtin_fmaxf(__builtin_fmaxf(m, lo_f(w)), hi_f(w));
      }
    m = dpp_max(m);
    if (m == -INFINITY) return -INFINITY;
    c = m * kLog2e;
    s = row16_sum(sum_shifted<VPL>(v, -c));
  }
  return c + log2f(s);  // -inf for a row with no active element
}

// alpha and S sums of this thread's vectors; m[k] gets the indicator byte of
// vector k (bit j: element j has z' < y').
template <int VPL>
__device__ inline float2 alpha_core(const Slice<VPL> &b, float lz2, float ly2, uint32_t (&mk)[VPL]) {
  float al = 0.f, ss = 0.f, nz = -lz2, ny = -ly2;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 7; j >= 0; --j) {  // element j ends up in bit j
      const uint32_t wz = word(b.z[k], j >> 1), wy = word(b.y[k], j >> 1);
      const float za = fmaf((j & 1) ? hi_q(wz) : lo_q(wz), kLog2e, nz);
      const float yb = fmaf((j & 1) ? hi_q(wy) : lo_q(wy), kLog2e, ny);
      const float e = __builtin_amdgcn_exp2f(fminf(za, yb));
      // in = za < yb; t = in ? e : 0; m = 2 m + in (the carry-in is the compare)
      float t;
      asm("v_cmp_lt_f32 vcc, %2, %3\n\t"
          "v_cndmask_b32 %1, 0, %4, vcc\n\t"
          "v_addc_co_u32 %0, vcc, %0, %0, vcc"
          : "+v"(m), "=&v"(t)
          : "v"(za), "v"(yb), "v"(e)
          : "vcc");
      al += e;
      ss += t;
    }
    mk[k] = m;
    // one vector at a time: the next vector's work depends on this vector's sums,
    // so the scheduler cannot hoist every compare ahead of the exponentials
    asm volatile("" : "+v"(al), "+v"(ss), "+v"(nz), "+v"(ny));
  }
  return make_float2(al, ss);
}

// alpha_core, with the indicator bytes stored through a buffer resource whose
// range is this member's slice of the bitmask row (stores of lanes past the
// slice are dropped by the hardware).
template <int VPL>
__device__ inline float2 team_alpha(const Slice<VPL> &b, float lz2, float ly2,
                                    __amdgpu_buffer_rsrc_t brow, uint32_t tl) {
  uint32_t mk[VPL];
  const float2 r = alpha_core<VPL>(b, lz2, ly2, mk);
#pragma unroll
  for (int k = 0; k < VPL; ++k) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)mk[k], brow, tl, k * kTeamData, 0);
  return r;
}

__device__ inline unsigned long long pack_slot(float lz, float ly) {
  if (lz != lz) lz = __uint_as_float(0x7fc00000u);  // canonical NaN, never the empty pattern
  if (ly != ly) ly = __uint_as_float(0x7fc00000u);
  return ((unsigned long long)__float_as_uint(ly) << 32) | __float_as_uint(lz);
}

struct TeamCtx {
  int64_t vb;          // first vector of this member's slice
  uint32_t n;          // vectors in the slice
  uint32_t voff;       // byte offset of this thread's first vector in a row
  int64_t r0, nr;      // first row of the team, rows of the team (stride n_teams)
  int mem, team;
};

struct TeamShared {
  float2 w[2][kTeamRows];        // 16-lane row (lse2 z, lse2 y) of a logit row, by row parity
  float2 as[2][kTeamRows];       // 16-lane row (alpha, S) of a logit row, by row parity
  float2 l[4];                   // logit row (lse2 z, lse2 y), by row mod 4
};

// Exchange of a row (sync wave), in two halves a step apart. publish: merge
// the wave values into the member's and store it into the row's slot.
__device__ inline void team_publish(const TeamArgs &a, const TeamCtx &c, int64_t r, int par,
                                    const TeamShared &sh) {
  const int lane = threadIdx.x & 63;
  float2 p = make_float2(-INFINITY, -INFINITY);
  if (lane < kTeamRows) p = sh.w[par][lane];
  const float mz = wave_lse2(p.x), my = wave_lse2(p.y);
  if (lane == 0)
    __hip_atomic_store(a.xchg + r * a.T + c.mem, pack_slot(mz, my), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// collect: poll the row's slots until every member's is written, merge them in
// member order into sh.l[slot]; member 0 also stores the row's values. False
// if the poll timed out (or another team's did).
__device__ inline bool team_collect(const TeamArgs &a, const TeamCtx &c, int64_t r, int slot,
                                    TeamShared &sh) {
  const int lane = threadIdx.x & 63, T = a.T;
  const unsigned long long *slots = a.xchg + r * T;
  unsigned long long v = kSlotEmpty;
  unsigned spins = 0;
  for (;;) {
    if (lane < T && v == kSlotEmpty)
      v = __hip_atomic_load(slots + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!__any(lane < T && v == kSlotEmpty)) break;
    unsigned bad = 0;
    if (lane == 63) bad = __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__shfl(bad, 63) != 0u || ++spins > kTeamSpinLimit) {
      if (lane == 0) __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  const float gz = lane < T ? __uint_as_float((uint32_t)v) : -INFINITY;
  const float gy = lane < T ? __uint_as_float((uint32_t)(v >> 32)) : -INFINITY;
  const float lz2 = wave_lse2(gz), ly2 = wave_lse2(gy);
  if (lane == 0) {
    sh.l[slot] = make_float2(lz2, ly2);
    if (c.mem == 0) {
      a.lse_q2[r] = lz2;
      a.lse_p2[r] = ly2;
    }
  }
  return true;
}

// The member's (alpha, S) of a row from the wave values (sync wave).
__device__ inline void team_flush(const TeamArgs &a, const TeamCtx &c, int64_t r, int par,
                                  const TeamShared &sh) {
  const int lane = threadIdx.x & 63;
  float2 q = make_float2(0.f, 0.f);
  if (lane < kTeamRows) q = sh.as[par][lane];
  q.x = dpp_sum(q.x);
  q.y = dpp_sum(q.y);
  if (lane == 0) a.part[r * a.T + c.mem] = q;
}

// Pass 1 of row i in `cur` (if the team has a row i) and the step's workgroup
// barrier, in a data wave.
template <int VPL>
__device__ inline void data_pass1(Slice<VPL> &cur, const TeamCtx &c, int64_t i, TeamShared &sh,
                                  int wv, uint32_t tl, float2 shift) {
  if (i < c.nr) {
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if ((uint32_t)((k + 1) * kTeamData) > c.n && tl + (uint32_t)(k * kTeamData) >= c.n) {
        cur.z[k] = make_uint4(kNegInf2, kNegInf2, kNegInf2, kNegInf2);
        cur.y[k] = cur.z[k];
      }
    const float lz = rows_lse2_of<VPL>(cur.z, true, shift.x);
    const float ly = rows_lse2_of<VPL>(cur.y, false, shift.y);
    if ((threadIdx.x & 15) == 0) sh.w[i & 1][wv * 4 + ((threadIdx.x & 63) >> 4)] = make_float2(lz, ly);
  }
  __syncthreads();
}

// Step i >= 2 of the pipeline in a data wave: pass 1 of row i in `cur`, the
// barrier, pass 2 of row i - 2 in `old`, then the loads of row i + 2 into `old`.
// Steps past the team's rows still issue the same memory operations, through
// empty buffer ranges that read and write nothing, so the loop has no branch
// around a memory operation and no early exit: the compiler's wait counts then
// see the true age of each buffer's loads (later buffers' loads stay in flight
// while a row is worked on).
template <int VPL>
__device__ inline void data_step(Slice<VPL> &cur, Slice<VPL> &old, const TeamArgs &a,
                                 const TeamCtx &c, int64_t i, TeamShared &sh, int wv) {
  // Slice-local vector index of this thread; laundered so that the per-vector
  // slice tests are made here rather than kept in scalar registers across steps.
  uint32_t tl = threadIdx.x;
  asm volatile("" : "+v"(tl));
  // the shift of pass 1: the log-sum-exps of row i - 3, the latest this step can see
  data_pass1<VPL>(cur, c, i, sh, wv, tl, i >= 3 ? sh.l[(i - 3) & 3] : make_float2(-INFINITY, -INFINITY));
  const int64_t r = c.r0 + i * a.n_teams;
  const bool has2 = i - 2 < c.nr;  // row i - 2 is one of the team's
  const float2 l = sh.l[(i - 2) & 3];
  const __amdgpu_buffer_rsrc_t brow =
      row_rsrc(has2 ? a.bits + (r - 2 * a.n_teams) * a.bits_row + c.vb : a.bits, has2 ? c.n : 0u);
  float2 as = team_alpha<VPL>(old, l.x, l.y, brow, tl);
  as.x = row16_sum(as.x);
  as.y = row16_sum(as.y);
  if ((threadIdx.x & 15) == 0) sh.as[i & 1][wv * 4 + ((threadIdx.x & 63) >> 4)] = as;
  team_load<VPL>(old, a, r + 2 * a.n_teams, c.voff, i + 2 < c.nr);
}

// The data waves and the sync wave run separate loops (the branch is uniform
// per wave) that meet at the same workgroup barriers, one per step; keeping the
// two codes apart also keeps the compiler from waiting on the data waves'
// in-flight loads where the paths would otherwise merge.
//
// Pipeline, four row buffers A, B, C, D (row i in buffer i % 4):
//   data step i:  pass 1 of row i | barrier | pass 2 of row i - 2, then the
//                 loads of row i + 2 into the buffer row i - 2 has freed;
//   sync step i:  barrier | (alpha, S) of row i - 3 to part | publish row i |
//                 collect row i - 1 (whose slots the other members wrote in
//                 their step i - 1, so the poll rarely waits).
// A row's log-sum-exps are ready one step before its pass 2 needs them. The
// steps from 2 on run in groups of four (one per buffer rotation), the last
// group padded with steps that have no row. A failed exchange only raises the
// status word (the results are then NaN); every wave still runs all steps, so
// the barriers always pair up.
template <int VPL>
__global__ __launch_bounds__(kTeamThreads) void e2etv_stats_team_kernel(TeamArgs a) {
  __shared__ TeamShared sh;
  TeamCtx c;
  c.team = blockIdx.x / a.T;
  c.mem = blockIdx.x % a.T;
  if (c.team >= a.n_teams) return;
  c.vb = a.V8 * c.mem / a.T;
  c.n = (uint32_t)(a.V8 * (c.mem + 1) / a.T - c.vb);
  c.voff = (uint32_t)((c.vb + threadIdx.x) * 16);
  c.r0 = c.team;
  c.nr = (a.R - c.team + a.n_teams - 1) / a.n_teams;
  if (c.nr <= 0) return;
  const int64_t last = 4 * ((c.nr + 3) / 4) + 1;  // final step: steps 2..last fill whole groups
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv < kTeamDataWaves) {
    Slice<VPL> A, B, C, D;
    team_load<VPL>(A, a, c.r0, c.voff, true);
    team_load<VPL>(B, a, c.r0 + a.n_teams, c.voff, c.nr > 1);
    uint32_t tl = threadIdx.x;
    asm volatile("" : "+v"(tl));
    // steps 0 and 1: pass 1 only, and the loads of rows 2 and 3
    const float2 none = make_float2(-INFINITY, -INFINITY);
    data_pass1<VPL>(A, c, 0, sh, wv, tl, none);
    team_load<VPL>(C, a, c.r0 + 2 * a.n_teams, c.voff, c.nr > 2);
    data_pass1<VPL>(B, c, 1, sh, wv, tl, none);
    team_load<VPL>(D, a, c.r0 + 3 * a.n_teams, c.voff, c.nr > 3);
    for (int64_t i = 2; i <= last; i += 4) {
      data_step<VPL>(C, A, a, c, i, sh, wv);
      data_step<VPL>(D, B, a, c, i + 1, sh, wv);
      data_step<VPL>(A, C, a, c, i + 2, sh, wv);
      data_step<VPL>(B, D, a, c, i + 3, sh, wv);
    }
    __syncthreads();
  } else {
    // The sync wave's work is a short dependent chain that the data waves'
    // steady compute would otherwise crowd out on its SIMD; it issues first.
    __builtin_amdgcn_s_setprio(3);
    bool ok = true;
    for (int64_t i = 0; i <= last; ++i) {
      const int64_t r = c.r0 + i * a.n_teams;
      __syncthreads();
      if (i >= 3 && i - 3 < c.nr) team_flush(a, c, r - 3 * a.n_teams, (int)((i - 3) & 1), sh);
      if (i < c.nr) team_publish(a, c, r, (int)(i & 1), sh);
      if (ok && i >= 1 && i - 1 < c.nr) ok = team_collect(a, c, r - a.n_teams, (int)((i - 1) & 3), sh);
    }
    __syncthreads();
    if (c.nr + 2 > last)  // row nr - 1 had no step i = nr + 2 to flush it
      team_flush(a, c, c.r0 + (c.nr - 1) * a.n_teams, (int)((c.nr - 1) & 1), sh);
  }
}

// ---------------------------------------------------------------------------
// Fused statistics and gradient (bf16 rows, length a multiple of 8, and every
// branch short enough that its rows fall in two consecutive steps of the team
// pipeline: W_b - 1 <= n_teams). Without a gradient buffer the same kernel
// runs with its gradient stores dropped, so alpha and L do not depend on
// whether the gradient is asked for.
//
// The team pipeline above, extended by a third exchange and a write stage, so
// that every logit is read once and every gradient element written once
// (8 bytes per element): a member keeps the draft words and the indicator bits
// of its slice of a row after pass 2, and three steps later, once the partials
// of every row of the row's branch are published, writes the gradient
//   g = c_s q (1[z' < y'] - S_s) = (bit ? c_s (1 - S_s) : -c_s S_s) 2^z'
// straight from registers. Rows are numbered r = team + i n_teams, so the rows
// of a branch sit in one step or two adjacent ones.
//   data step i:  pass 1 of row i | barrier | pass 2 of row i - 2 (bits and
//                 draft words kept; the last wave through it stores the
//                 member's (alpha, S) partial of the row into its slot) |
//                 gradient of row i - 5 | loads of row i + 2
//   sync step i:  barrier | publish row i | collect row i - 1 and the
//                 coefficient of row i - 4 (one poll)
// The coefficient of row g polls the partial slots of every row of g's
// branch (rows of g's step and the next, flushed during data step g + 3, a
// step before the poll), adds each row's
// partials in member order, forms A and G in float64 as the scan kernel does
// and leaves (lse2 z, c (1 - S), -c S) of row g in LDS for the next data step.
// Member 0 of a row stores its alpha; member 0 of a branch's first row stores
// the branch's sum of prefix products, which a one-workgroup kernel adds in
// branch order after this one. Partial slots are 64-bit words written once by
// agent-scope atomic stores and cleared to all-ones before the launch.

constexpr int kFuseMaxVpl = 2;  // four row buffers and four held draft slices per lane
constexpr int kFuseRowCap = 2048;  // rows per team whose branch extents sit in LDS

struct FuseArgs {
  TeamArgs t;
  float *grad;                   // [R][V] float32, or null (no gradient)
  float *alpha;                  // [R]
  const int32_t *step_off;       // [B + 1]
  const int32_t *step_branch;    // [R]
  double *branch_sum;            // [B]
  float w;                       // loss normaliser
};

struct FuseShared {
  TeamShared t;
  unsigned cnt[2];                               // data waves through pass 2, by step parity
  float4 gc[4];                                  // row (lse2 z, c (1 - S), -c S, -), by row mod 4
  unsigned long long pp[64 * kTeamMax];          // a branch's partial slots, row-major [W][T]
  int4 rows[kFuseRowCap];                        // the team's k-th row: (branch, first step, width, -)
};

__device__ inline unsigned long long pack_pair(float a, float b) { return pack_slot(a, b); }

// The member's (alpha, S) of a row, into the row's slot for this member.
__device__ inline void fuse_flush(const FuseArgs &a, const TeamCtx &c, int64_t r, int par,
                                  const FuseShared &sh) {
  const int lane = threadIdx.x & 63;
  float2 q = make_float2(0.f, 0.f);
  if (lane < kTeamRows) q = sh.t.as[par][lane];
  q.x = dpp_sum(q.x);
  q.y = dpp_sum(q.y);
  unsigned long long *slot = reinterpret_cast<unsigned long long *>(a.t.part) + r * a.t.T + c.mem;
  if (lane == 0) __hip_atomic_store(slot, pack_pair(q.x, q.y), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sync work of step i after the flush and the publish: collect row i - 1 (if
// `col`) and the coefficient of row g = i - 4 (if `coef`). The slots of both
// are polled together, so a step costs one round trip to the coherence point.
// The coefficient polls the partial slots of every row of g's branch, adds
// each row's partials in member order, forms A and G in float64 as the scan
// kernel does and leaves (lse2 z, c (1 - S), -c S) of row g in LDS for the next
// data step. False on a poll timeout.
__device__ inline bool fuse_sync(const FuseArgs &a, const TeamCtx &c, int64_t i, bool col, bool coef,
                                 FuseShared &sh) {
  const int lane = threadIdx.x & 63, T = a.t.T;
  const int64_t n = a.t.n_teams;
  const int64_t rc = c.r0 + (i - 1) * n, g = c.r0 + (i - 4) * n;
  int b = 0, s0 = 0, W = 0, WT = 0;
  if (coef) {
    const int4 e = sh.rows[i - 4];
    b = e.x;
    s0 = e.y;
    W = e.z;
    WT = W * T;
  }
  const unsigned long long *xs = a.t.xchg + rc * T;
  const unsigned long long *ps = reinterpret_cast<const unsigned long long *>(a.t.part) + (int64_t)s0 * T;
  constexpr int kPer = kTeamMax;  // slots per lane: W T <= 64 kTeamMax
  unsigned long long vx = kSlotEmpty, v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) v[k] = kSlotEmpty;
  const bool wx = col && lane < T;
  unsigned spins = 0;
  for (;;) {
    if (wx && vx == kSlotEmpty) vx = __hip_atomic_load(xs + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = lane + 64 * k;
      if (64 * k < WT && e < WT && v[k] == kSlotEmpty)
        v[k] = __hip_atomic_load(ps + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    bool missing = wx && vx == kSlotEmpty;
#pragma unroll
    for (int k = 0; k < kPer; ++k) missing |= (lane + 64 * k < WT) && v[k] == kSlotEmpty;
    if (!__any(missing)) break;
    unsigned bad = 0;
    if (lane == 63) bad = __hip_atomic_load(a.t.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__shfl(bad, 63) != 0u || ++spins > kTeamSpinLimit) {
      if (lane == 0) __hip_atomic_store(a.t.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (col) {  // row i - 1: merge the members' log-sum-exps in member order
    const float gz = wx ? __uint_as_float((uint32_t)vx) : -INFINITY;
    const float gy = wx ? __uint_as_float((uint32_t)(vx >> 32)) : -INFINITY;
    const float lz2 = wave_lse2(gz), ly2 = wave_lse2(gy);
    if (lane == 0) sh.t.l[(i - 1) & 3] = make_float2(lz2, ly2);
  }
  if (!coef) return true;
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (lane + 64 * k < WT) sh.pp[lane + 64 * k] = v[k];
  float al = 0.f, ss = 0.f;
  if (lane < W) {
    for (int j = 0; j < T; ++j) {
      const unsigned long long x = sh.pp[lane * T + j];
      al += __uint_as_float((uint32_t)x);
      ss += __uint_as_float((uint32_t)(x >> 32));
    }
  }
  // lane i: A_{i-1} = prod_{j<i} alpha_j (ascending), G_i = 1 + alpha_{i+1} G_{i+1};
  // alpha_j reaches every lane through a scalar read of lane j
  const double ad = al;
  double A = 1.0, G = 1.0;
  for (int j = 0; j < W; ++j) {
    const double aj = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), j));
    if (j < lane) A *= aj;
  }
  for (int j = W - 1; j > 0; --j) {
    const double aj = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), j));
    if (j > lane) G = 1.0 + aj * G;
  }
  const float cf = (float)(-(double)a.w * A * G);
  const int gl = (int)(g - s0);
  const float cg = __shfl(cf, gl), sg = __shfl(ss, gl);
  if (lane == 0) {
    const float lz2 = sh.t.l[(i - 4) & 3].x;
    sh.gc[(i - 4) & 3] = make_float4(lz2, cg * (1.f - sg), -cg * sg, 0.f);
  }
  if (c.mem == 0) {
    if (lane == gl) a.alpha[g] = al;
    if (gl == 0) {  // the branch's first row: its sum of prefix products
      double sumA = lane < W ? A * ad : 0.0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) sumA += __shfl_xor(sumA, off);
      if (lane == 0) a.branch_sum[b] = sumA;
    }
  }
  return true;
}

// Gradient of one row slice from the held draft words and indicator bits.
template <int VPL>
__device__ inline void fuse_grad(const uint4 (&zh)[VPL], uint32_t bits, float4 gc,
                                 __amdgpu_buffer_rsrc_t grow, uint32_t tl) {
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t wz = word(zh[k], j >> 1);
      const float q = __builtin_amdgcn_exp2f(fmaf((j & 1) ? hi_f(wz) : lo_f(wz), kLog2e, -gc.x));
      g[j] = ((bits >> (8 * k + j)) & 1u ? gc.y : gc.z) * q;
    }
    const uint32_t off = (tl + (uint32_t)(k * kTeamData)) * 32u;
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]), __float_as_uint(g[3])},
        grow, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(g[4]), __float_as_uint(g[5]), __float_as_uint(g[6]), __float_as_uint(g[7])},
        grow, off + 16u, 0, 0);
  }
}

// Data step i >= 2 of the fused pipeline (see above). `cur` holds row i,
// `old` row i - 2 (then the loads of row i + 2); (zw, bw) receive row i - 2's
// draft words and bits, (zr, br) hold row i - 5's.
template <int VPL>
__device__ inline void fuse_step(Slice<VPL> &cur, Slice<VPL> &old, uint4 (&zw)[VPL], uint32_t &bw,
                                 const uint4 (&zr)[VPL], uint32_t br, const FuseArgs &a,
                                 const TeamCtx &c, int64_t i, FuseShared &sh, int wv) {
  uint32_t tl = threadIdx.x;
  asm volatile("" : "+v"(tl));
  data_pass1<VPL>(cur, c, i, sh.t, wv, tl, i >= 3 ? sh.t.l[(i - 3) & 3] : make_float2(-INFINITY, -INFINITY));
  const int64_t n = a.t.n_teams;
  const int64_t r = c.r0 + i * n;
  const float2 l = sh.t.l[(i - 2) & 3];
  uint32_t mk[VPL];
  float2 as = alpha_core<VPL>(old, l.x, l.y, mk);
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    bits |= mk[k] << (8 * k);
    zw[k] = old.z[k];
  }
  bw = bits;
  as.x = row16_sum(as.x);
  as.y = row16_sum(as.y);
  if ((threadIdx.x & 15) == 0) sh.t.as[i & 1][wv * 4 + ((threadIdx.x & 63) >> 4)] = as;
  // the last data wave through pass 2 flushes the member's (alpha, S) of row
  // i - 2 and rearms the counter for step i + 2
  unsigned prev = 0;
  if ((threadIdx.x & 63) == 0)
    prev = __hip_atomic_fetch_add(&sh.cnt[i & 1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (__builtin_amdgcn_readfirstlane(prev) == (unsigned)kTeamDataWaves - 1) {
    if (i - 2 < c.nr) fuse_flush(a, c, r - 2 * n, (int)(i & 1), sh);
    if ((threadIdx.x & 63) == 0) sh.cnt[i & 1] = 0u;
  }
  const bool hasg = i >= 5 && i - 5 < c.nr && a.grad != nullptr;
  const int64_t V = a.t.V8 * 8;
  const __amdgpu_buffer_rsrc_t grow =
      row_rsrc(hasg ? a.grad + (r - 5 * n) * V + c.vb * 8 : a.grad, hasg ? c.n * 32u : 0u);
  fuse_grad<VPL>(zr, br, sh.gc[(i - 5) & 3], grow, tl);
  team_load<VPL>(old, a.t, r + 2 * n, c.voff, i + 2 < c.nr);
}

template <int VPL>
__global__ __launch_bounds__(kTeamThreads) void e2etv_fused_team_kernel(FuseArgs a) {
  __shared__ FuseShared sh;
  TeamCtx c;
  c.team = blockIdx.x / a.t.T;
  c.mem = blockIdx.x % a.t.T;
  if (c.team >= a.t.n_teams) return;
  c.vb = a.t.V8 * c.mem / a.t.T;
  c.n = (uint32_t)(a.t.V8 * (c.mem + 1) / a.t.T - c.vb);
  c.voff = (uint32_t)((c.vb + threadIdx.x) * 16);
  c.r0 = c.team;
  c.nr = (a.t.R - c.team + a.t.n_teams - 1) / a.t.n_teams;
  if (c.nr <= 0) return;
  const int64_t last = 4 * ((c.nr + 6) / 4) + 1;  // steps 2..last fill whole groups; last >= nr + 4
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x < 2) sh.cnt[threadIdx.x] = 0u;  // first used after the barrier of step 2
  if (wv < kTeamDataWaves) {
    Slice<VPL> A, B, C, D;
    uint4 Z0[VPL], Z1[VPL], Z2[VPL], Z3[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) Z0[k] = Z1[k] = Z2[k] = Z3[k] = make_uint4(0, 0, 0, 0);
    uint32_t b0 = 0, b1 = 0, b2 = 0, b3 = 0;
    team_load<VPL>(A, a.t, c.r0, c.voff, true);
    team_load<VPL>(B, a.t, c.r0 + a.t.n_teams, c.voff, c.nr > 1);
    uint32_t tl = threadIdx.x;
    asm volatile("" : "+v"(tl));
    const float2 none = make_float2(-INFINITY, -INFINITY);
    data_pass1<VPL>(A, c, 0, sh.t, wv, tl, none);
    team_load<VPL>(C, a.t, c.r0 + 2 * a.t.n_teams, c.voff, c.nr > 2);
    data_pass1<VPL>(B, c, 1, sh.t, wv, tl, none);
    team_load<VPL>(D, a.t, c.r0 + 3 * a.t.n_teams, c.voff, c.nr > 3);
    // row i in buffer i % 4; row i - 2's draft slice held in Z[(i - 2) % 4]
    for (int64_t i = 2; i <= last; i += 4) {
      fuse_step<VPL>(C, A, Z0, b0, Z1, b1, a, c, i, sh, wv);
      fuse_step<VPL>(D, B, Z1, b1, Z2, b2, a, c, i + 1, sh, wv);
      fuse_step<VPL>(A, C, Z2, b2, Z3, b3, a, c, i + 2, sh, wv);
      fuse_step<VPL>(B, D, Z3, b3, Z0, b0, a, c, i + 3, sh, wv);
    }
    __syncthreads();
  } else {
    __builtin_amdgcn_s_setprio(3);
    // the branch extent of every row of the team, once, so that no poll waits
    // behind a dependent pair of global loads
    for (int64_t k = threadIdx.x & 63; k < c.nr; k += 64) {
      const int b = a.step_branch[c.r0 + k * a.t.n_teams];
      const int s0 = a.step_off[b];
      sh.rows[k] = make_int4(b, s0, a.step_off[b + 1] - s0, 0);
    }
    bool ok = true;
    for (int64_t i = 0; i <= last; ++i) {
      const int64_t r = c.r0 + i * a.t.n_teams;
      __syncthreads();
      if (i < c.nr) team_publish(a.t, c, r, (int)(i & 1), sh.t);
      const bool col = i >= 1 && i - 1 < c.nr, coef = i >= 4 && i - 4 < c.nr;  // wave-uniform
      if (ok && (col || coef)) ok = fuse_sync(a, c, i, col, coef, sh);
    }
    __syncthreads();
  }
}

// L = 1 - w * sum of the branch sums in branch order (one workgroup, after the
// fused kernel); a raised status word makes L NaN.
__global__ __launch_bounds__(1024) void e2etv_loss_kernel(const double *__restrict__ branch_sum,
                                                          int32_t n_branches, const unsigned *__restrict__ status,
                                                          float w, float *__restrict__ alpha, int64_t R,
                                                          float *__restrict__ loss) {
  __shared__ double red[16];
  const bool failed = *status != 0u;
  if (failed)
    for (int64_t s = threadIdx.x; s < R; s += blockDim.x) alpha[s] = NAN;
  double t = 0.0;
  for (int k = threadIdx.x; k < n_branches; k += blockDim.x) t += branch_sum[k];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) t += __shfl_xor(t, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) tot += red[k];
    loss[0] = failed ? NAN : (float)(1.0 - (double)w * tot);
  }
}

// Slots to the empty pattern, the status word and the scan ticket to zero,
// before a team launch.
__global__ void e2etv_team_clear(unsigned long long *xchg, int64_t n, unsigned *status) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    xchg[i] = kSlotEmpty;
  if (blockIdx.x == 0 && threadIdx.x < 2) status[threadIdx.x] = 0u;
}

// Exchange slots and partial slots to the empty pattern, the status word to
// zero, before a fused launch.
__global__ void e2etv_fuse_clear(unsigned long long *xchg, unsigned long long *part, int64_t n,
                                 unsigned *status) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    xchg[i] = kSlotEmpty;
    part[i] = kSlotEmpty;
  }
  if (blockIdx.x == 0 && threadIdx.x < 2) status[threadIdx.x] = 0u;
}

// One wave per branch and one lane per step (a branch has at most 64 steps).
// Each lane adds its row's member partials in member order into alpha_s and
// S_s; the branch's alphas are then broadcast lane by lane in float64 so that
// lane i forms A_{i-1} = prod_{j<i} alpha_j (ascending order) and
// G_i = 1 + alpha_{i+1} G_{i+1} with G_W = 1, hence c_i = -w A_{i-1} G_i with
// no division. The branch's sum of A_j is a fixed butterfly over the lanes.
// The last workgroup to take a ticket (cleared by the statistics kernels) adds
// the branch sums in branch order and writes L = 1 - w * sum. A raised status
// word (a statistics team exchange that timed out) makes alpha and L NaN.
constexpr int kScanWaves = 16;
__global__ __launch_bounds__(kScanWaves * 64) void e2etv_scan_kernel(
    const int32_t *__restrict__ step_off, int32_t n_branches, const float2 *__restrict__ part,
    int32_t team, const unsigned *__restrict__ status, float w, float *__restrict__ alpha,
    float *__restrict__ S, float *__restrict__ coef, double *__restrict__ branch_sum,
    unsigned *__restrict__ ticket, float *__restrict__ loss) {
  __shared__ double red[kScanWaves];
  __shared__ bool is_last;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = blockIdx.x * kScanWaves + wv;
  const bool failed = status != nullptr && *status != 0u;
  if (b < n_branches) {
    const int s0 = step_off[b], n = step_off[b + 1] - s0;
    float al = 0.f, ss = 0.f;
    if (lane < n) {
      const float2 *pp = part + (int64_t)(s0 + lane) * team;
      for (int j = 0; j < team; ++j) {
        const float2 p = pp[j];
        al += p.x;
        ss += p.y;
      }
      alpha[s0 + lane] = failed ? NAN : al;
      S[s0 + lane] = ss;
    }
    const double ad = al;
    double A = 1.0, G = 1.0;
    for (int j = 0; j < n; ++j) {
      const double aj = __shfl(ad, j);
      if (j < lane) A *= aj;
    }
    for (int j = n - 1; j > 0; --j) {
      const double aj = __shfl(ad, j);
      if (j > lane) G = 1.0 + aj * G;
    }
    double sumA = 0.0;
    if (lane < n) {
      coef[s0 + lane] = (float)(-(double)w * A * G);
      sumA = A * ad;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) sumA += __shfl_xor(sumA, off);
    if (lane == 0) {
      branch_sum[b] = sumA;
      __threadfence();  // the branch sum is visible to whichever workgroup finishes last
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) is_last = atomicAdd(ticket, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  double t = 0.0;
  for (int k = threadIdx.x; k < n_branches; k += blockDim.x) t += branch_sum[k];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) t += __shfl_xor(t, off);
  if (lane == 0) red[wv] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int k = 0; k < kScanWaves; ++k) tot += red[k];
    loss[0] = failed ? NAN : (float)(1.0 - (double)w * tot);
    *ticket = 0u;
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kGradThreads) void e2etv_grad_kernel(
    const T *__restrict__ draft, const T *__restrict__ teacher, int64_t V,
    const float *__restrict__ lse_q2, const float *__restrict__ lse_p2,
    const float *__restrict__ S, const float *__restrict__ coef, float *__restrict__ grad,
    const uint8_t *__restrict__ bits, int64_t bits_row, int32_t chunks_per_row) {
  const int64_t row = blockIdx.x / chunks_per_row;
  const int64_t chunk = blockIdx.x % chunks_per_row;
  const float lz2 = lse_q2[row], ly2 = lse_p2[row], c = coef[row], ss = S[row];
  const float cin = c * (1.f - ss), cout = -c * ss;  // coefficient inside / outside {q < p}
  const T *z = draft + row * V;
  const T *y = teacher + row * V;
  float *g = grad + row * V;
  if (VEC) {
    // kGradVecs 8-element vectors per thread, block-strided so each load is contiguous per wave;
    // the set {q < p} comes from the statistics pass's bitmask, so the teacher row is not read
    const uint8_t *brow = bits + row * bits_row;
    float a[kGradVecs][8];
    uint32_t m[kGradVecs];
#pragma unroll
    for (int v = 0; v < kGradVecs; ++v) {
      const int64_t i = ((chunk * kGradVecs + v) * kGradThreads + threadIdx.x) * 8;
      if (i < V) {
        load8(z + i, a[v]);
        m[v] = brow[i / 8];
      }
    }
#pragma unroll
    for (int v = 0; v < kGradVecs; ++v) {
      const int64_t i = ((chunk * kGradVecs + v) * kGradThreads + threadIdx.x) * 8;
      if (i >= V) continue;
      float r[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float za = fmaf(sanitize(a[v][k]), kLog2e, -lz2);
        r[k] = ((m[v] >> k) & 1u ? cin : cout) * __builtin_amdgcn_exp2f(za);
      }
      float4 *gp = reinterpret_cast<float4 *>(g + i);
      gp[0] = make_float4(r[0], r[1], r[2], r[3]);
      gp[1] = make_float4(r[4], r[5], r[6], r[7]);
    }
  } else {
    const int64_t i0 = (chunk * kGradThreads + threadIdx.x) * 8 * kGradVecs;
    for (int64_t i = i0; i < i0 + 8 * kGradVecs && i < V; ++i) {
      const float za = fmaf(sanitize(load1(z + i)), kLog2e, -lz2);
      const float yb = fmaf(load1(y + i), kLog2e, -ly2);
      g[i] = (za < yb ? cin : cout) * __builtin_amdgcn_exp2f(za);
    }
  }
}

namespace {

constexpr int kTeamMaxVpl = 3;  // vectors per lane and array; three row buffers live per lane

struct TeamDevice {
  bool init = false;
  int cus = 0, coop = 0;
  int occ[kTeamMaxVpl + 1] = {};
  int fuse_occ[kFuseMaxVpl + 1] = {};
};

template <int VPL>
int team_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)e2etv_stats_team_kernel<VPL>,
                                                   kTeamThreads, 0) != hipSuccess)
    n = 0;
  return n;
}

template <int VPL>
int fuse_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)e2etv_fused_team_kernel<VPL>,
                                                   kTeamThreads, 0) != hipSuccess)
    n = 0;
  return n;
}

// Device properties and team-kernel occupancy, looked up once per device.
TeamDevice team_device(int dev) {
  static std::mutex mu;
  static TeamDevice cache[64];
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= 64) return TeamDevice{};
  TeamDevice &d = cache[dev];
  if (!d.init) {
    // a failed query leaves cus / coop at 0, which turns the team paths off
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) d.cus = 0;
    if (hipDeviceGetAttribute(&d.coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) d.coop = 0;
    d.occ[1] = team_occupancy<1>();
    d.occ[2] = team_occupancy<2>();
    d.occ[3] = team_occupancy<3>();
    d.fuse_occ[1] = fuse_occupancy<1>();
    d.fuse_occ[2] = fuse_occupancy<2>();
    d.init = true;
  }
  return d;
}

// Single-read statistics if the rows fit a team; *team = 0 if they do not.
hipError_t launch_team_stats(int64_t R, int64_t V, const void *draft, const void *teacher,
                             const E2etvWork &ws, hipStream_t s, int *team) {
  *team = 0;
  const int64_t V8 = V / 8;
  const int64_t per_member = (int64_t)kTeamData * kTeamMaxVpl;
  const int64_t T = (V8 + per_member - 1) / per_member;
  if (T < 1 || T > kTeamMax || V8 * 16 > INT32_MAX) return hipSuccess;
  const int vpl = (int)(((V8 + T - 1) / T + kTeamData - 1) / kTeamData);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const TeamDevice d = team_device(dev);
  if (!d.coop || d.cus < 1 || d.occ[vpl] < 1) return hipSuccess;
  const int64_t n_teams = std::min<int64_t>((int64_t)d.occ[vpl] * d.cus / T, R);
  if (n_teams < 1) return hipSuccess;
  const int64_t n_slots = R * T;
  hipLaunchKernelGGL(e2etv_team_clear, dim3((unsigned)std::min<int64_t>(256, (n_slots + 255) / 256)), dim3(256),
                     0, s, ws.xchg, n_slots, ws.status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  TeamArgs a;
  a.z = static_cast<const __bf16 *>(draft);
  a.y = static_cast<const __bf16 *>(teacher);
  a.R = R;
  a.V8 = V8;
  a.T = (int32_t)T;
  a.n_teams = (int32_t)n_teams;
  a.lse_q2 = ws.lse_q2;
  a.lse_p2 = ws.lse_p2;
  a.part = ws.part;
  a.bits = ws.bits;
  a.bits_row = ws.bits_row;
  a.xchg = ws.xchg;
  a.status = ws.status;
  void *args[] = {&a};
  static_assert(kTeamMaxVpl == 3, "one instantiation per vectors-per-lane count");
  const void *fn = vpl == 1   ? (const void *)e2etv_stats_team_kernel<1>
                   : vpl == 2 ? (const void *)e2etv_stats_team_kernel<2>
                              : (const void *)e2etv_stats_team_kernel<3>;
  e = hipLaunchCooperativeKernel(fn, dim3((unsigned)(n_teams * T)), dim3(kTeamThreads), args, 0, s);
  if (e != hipSuccess) return e;
  *team = (int)T;
  return hipSuccess;
}

// Fused statistics and gradient if the rows fit a team and every branch spans
// at most two pipeline steps; *done = false (nothing launched) otherwise.
// Shape of a fused launch: team size T, vectors per lane and team count.
struct FusePlan {
  int64_t T = 0, n_teams = 0;
  int vpl = 0;
};

// Whether bf16 rows of V (a multiple of 8) entries fit the fused pipeline on the
// current device: a row slice per member in registers, every branch within two
// pipeline steps (W_b - 1 <= team count) and the team's rows' branch extents in LDS.
hipError_t fuse_plan(const spec_tree_layout &L, int64_t V, FusePlan *p, bool *ok) {
  *ok = false;
  const int64_t R = L.n_steps;
  const int64_t V8 = V / 8;
  const int64_t per_member = (int64_t)kTeamData * kFuseMaxVpl;
  const int64_t T = (V8 + per_member - 1) / per_member;
  if (V % 8 != 0 || T < 1 || T > kTeamMax || V8 * 32 > INT32_MAX || L.max_branch_len > 64) return hipSuccess;
  const int vpl = (int)(((V8 + T - 1) / T + kTeamData - 1) / kTeamData);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const TeamDevice d = team_device(dev);
  if (!d.coop || d.cus < 1 || vpl < 1 || vpl > kFuseMaxVpl || d.fuse_occ[vpl] < 1) return hipSuccess;
  const int64_t n_teams = std::min<int64_t>((int64_t)d.fuse_occ[vpl] * d.cus / T, R);
  if (n_teams < 1 || (int64_t)L.max_branch_len - 1 > n_teams || (R + n_teams - 1) / n_teams > kFuseRowCap)
    return hipSuccess;
  p->T = T;
  p->n_teams = n_teams;
  p->vpl = vpl;
  *ok = true;
  return hipSuccess;
}

hipError_t launch_fused(const spec_tree_layout &L, int64_t V, const void *draft, const void *teacher,
                        float w, float *alpha, float *loss, float *grad, const E2etvWork &ws,
                        hipStream_t s, bool *done) {
  *done = false;
  const int64_t R = L.n_steps;
  const int64_t V8 = V / 8;
  FusePlan plan;
  bool ok = false;
  hipError_t e = fuse_plan(L, V, &plan, &ok);
  if (e != hipSuccess || !ok) return e;
  const int64_t T = plan.T, n_teams = plan.n_teams;
  const int vpl = plan.vpl;
  const int64_t n_slots = R * T;
  hipLaunchKernelGGL(e2etv_fuse_clear, dim3((unsigned)std::min<int64_t>(1024, (n_slots + 255) / 256)), dim3(256),
                     0, s, ws.xchg, reinterpret_cast<unsigned long long *>(ws.part), n_slots, ws.status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_clear");
  FuseArgs a;
  a.t.z = static_cast<const __bf16 *>(draft);
  a.t.y = static_cast<const __bf16 *>(teacher);
  a.t.R = R;
  a.t.V8 = V8;
  a.t.T = (int32_t)T;
  a.t.n_teams = (int32_t)n_teams;
  a.t.lse_q2 = ws.lse_q2;
  a.t.lse_p2 = ws.lse_p2;
  a.t.part = ws.part;
  a.t.bits = ws.bits;
  a.t.bits_row = ws.bits_row;
  a.t.xchg = ws.xchg;
  a.t.status = ws.status;
  a.grad = grad;
  a.alpha = alpha;
  a.step_off = L.step_off;
  a.step_branch = L.step_branch;
  a.branch_sum = ws.branch_sum;
  a.w = w;
  void *args[] = {&a};
  static_assert(kFuseMaxVpl == 2, "one instantiation per vectors-per-lane count");
  const void *fn = vpl == 1 ? (const void *)e2etv_fused_team_kernel<1> : (const void *)e2etv_fused_team_kernel<2>;
  e = hipLaunchCooperativeKernel(fn, dim3((unsigned)(n_teams * T)), dim3(kTeamThreads), args, 0, s);
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_fused");
  hipLaunchKernelGGL(e2etv_loss_kernel, dim3(1), dim3(1024), 0, s, ws.branch_sum, L.n_branches, ws.status,
                     w, alpha, R, loss);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_loss");
  *done = true;
  return hipSuccess;
}

template <typename T, bool VEC>
hipError_t launch_typed(const spec_tree_layout &L, int64_t V, const void *draft,
                        const void *teacher, float w, float *alpha, float *loss, float *grad,
                        const E2etvWork &ws, hipStream_t s) {
  const T *z = static_cast<const T *>(draft);
  const T *y = static_cast<const T *>(teacher);
  const int64_t R = L.n_steps;
  int team = 0;
  hipError_t e = hipSuccess;
  const unsigned *status = nullptr;
  if (std::is_same<T, __bf16>::value && VEC) {
    bool fused = false;
    e = launch_fused(L, V, draft, teacher, w, alpha, loss, grad, ws, s, &fused);
    if (e != hipSuccess || fused) return e;
  }
  // every other path keeps the {q < p} bitmask; a workspace carved without it
  // (the fused path's share only) cannot take them
  if (!ws.bits) return hipErrorInvalidValue;
  if (std::is_same<T, __bf16>::value && VEC) {
    e = launch_team_stats(R, V, draft, teacher, ws, s, &team);
    if (e != hipSuccess) return e;
    if (team) status = ws.status;
  }
  if (!team) {
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(R, cus));
    hipLaunchKernelGGL((e2etv_stats_kernel<T, VEC>), dim3((unsigned)grid), dim3(kStatThreads), 0, s,
                       z, y, R, V, ws.part, ws.lse_q2, ws.lse_p2, ws.bits, ws.bits_row, ws.status + 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    team = 1;
  }
  prof_mark(s, "e2etv_stats");
  hipLaunchKernelGGL(e2etv_scan_kernel, dim3((unsigned)((L.n_branches + kScanWaves - 1) / kScanWaves)),
                     dim3(kScanWaves * 64), 0, s, L.step_off, L.n_branches, ws.part, team, status, w,
                     alpha, ws.S, ws.coef, ws.branch_sum, ws.status + 1, loss);
  e = hipGetLastError();
  if (e != hipSuccess || !grad) return e;
  prof_mark(s, "e2etv_scan");
  const int64_t per_block = (int64_t)kGradThreads * 8 * kGradVecs;
  const int64_t chunks = (V + per_block - 1) / per_block;
  if (chunks * R > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((e2etv_grad_kernel<T, VEC>), dim3((unsigned)(chunks * R)), dim3(kGradThreads),
                     0, s, z, y, V, ws.lse_q2, ws.lse_p2, ws.S, ws.coef, grad, ws.bits, ws.bits_row,
                     (int32_t)chunks);
  e = hipGetLastError();
  prof_mark(s, "e2etv_grad");
  return e;
}

}  // namespace

hipError_t e2etv_takes_fused_path(const spec_tree_layout &L, int64_t V, spec_dtype dtype, bool *fused) {
  *fused = false;
  if (dtype != SPEC_BF16 || V % 8 != 0) return hipSuccess;
  FusePlan plan;
  return fuse_plan(L, V, &plan, fused);
}

hipError_t launch_e2etv(const spec_tree_layout &L, int64_t V, spec_dtype dtype, const void *draft,
                        const void *teacher, float w, float *alpha, float *loss, float *grad,
                        const E2etvWork &ws, hipStream_t s) {
  const bool vec = (V % 8) == 0;
  if (dtype == SPEC_BF16)
    return vec ? launch_typed<__bf16, true>(L, V, draft, teacher, w, alpha, loss, grad, ws, s)
               : launch_typed<__bf16, false>(L, V, draft, teacher, w, alpha, loss, grad, ws, s);
  return vec ? launch_typed<float, true>(L, V, draft, teacher, w, alpha, loss, grad, ws, s)
             : launch_typed<float, false>(L, V, draft, teacher, w, alpha, loss, grad, ws, s);
}

hipError_t launch_e2etv_tail(const spec_tree_layout &L, int64_t V, spec_dtype dtype, const void *draft,
                             float w, int team, float *alpha, float *loss, float *grad,
                             const E2etvWork &ws, hipStream_t s) {
  hipLaunchKernelGGL(e2etv_scan_kernel, dim3((unsigned)((L.n_branches + kScanWaves - 1) / kScanWaves)),
                     dim3(kScanWaves * 64), 0, s, L.step_off, L.n_branches, ws.part, team,
                     (const unsigned *)nullptr, w, alpha, ws.S, ws.coef, ws.branch_sum,
                     ws.status + 1, loss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !grad) return e;
  prof_mark(s, "e2etv_scan");
  const int64_t R = L.n_steps;
  const int64_t per_block = (int64_t)kGradThreads * 8 * kGradVecs;
  const int64_t chunks = (V + per_block - 1) / per_block;
  if (chunks * R > INT32_MAX || V % 8 != 0) return hipErrorInvalidValue;
  // the vector gradient path reads the draft row and the bitmask only
  if (dtype == SPEC_BF16) {
    const __bf16 *z = static_cast<const __bf16 *>(draft);
    hipLaunchKernelGGL((e2etv_grad_kernel<__bf16, true>), dim3((unsigned)(chunks * R)),
                       dim3(kGradThreads), 0, s, z, z, V, ws.lse_q2, ws.lse_p2, ws.S, ws.coef, grad,
                       ws.bits, ws.bits_row, (int32_t)chunks);
  } else {
    const float *z = static_cast<const float *>(draft);
    hipLaunchKernelGGL((e2etv_grad_kernel<float, true>), dim3((unsigned)(chunks * R)),
                       dim3(kGradThreads), 0, s, z, z, V, ws.lse_q2, ws.lse_p2, ws.S, ws.coef, grad,
                       ws.bits, ws.bits_row, (int32_t)chunks);
  }
  e = hipGetLastError();
  prof_mark(s, "e2etv_grad");
  return e;
}

}  // namespace spec
