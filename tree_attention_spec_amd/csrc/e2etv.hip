// E2E-TV surrogate, loss and gradient with respect to the draft logits.
//
// [SpecOPD notes page, "Equations"]: alpha_{b,i} = sum_v min(q_v, p_v) over the
// full vocabulary; L = 1 - (1/(BW)) sum_b sum_j prod_{i<=j} alpha_{b,i}; samples
// and the teacher are fixed when differentiating; teacher mass outside the draft
// support is kept. [SpecOPD notes page, "Inputs and code mapping"]: low
// precision is promoted to float32; NaN draft entries are inactive support.
//
// Three kernels on the caller's stream:
//   e2etv_stats  one workgroup per row: pass 1 streams the row for both
//                log-sum-exps (online max/sum per lane), pass 2 re-streams it for
//                alpha = sum 2^min(z', y') and S = sum over {z' < y'} of 2^z', where
//                z' = z*log2(e) - lse2(z) is log2 q (and y' likewise log2 p);
//   e2etv_scan   one workgroup: per branch the suffix sums G and prefix products
//                A give c_s = dL/d alpha_s = -w A_{i-1} G_i (no division), and the
//                loss is reduced in float64 in a fixed order;
//   e2etv_grad   grad[s,u] = c_s * q_u * (1[z'_u < y'_u] - S_s), written once.
// Every reduction has a fixed order, so results are bitwise reproducible. The
// strict test z' < y' is the same expression in all three places, so the set
// {q < p} used for S and for the gradient is the same set.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace spec {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStatThreads = 256;
constexpr int kGradThreads = 256;

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
    const T *__restrict__ draft, const T *__restrict__ teacher, int64_t V, float *__restrict__ alpha,
    float *__restrict__ S_out, float *__restrict__ lse_q2, float *__restrict__ lse_p2) {
  __shared__ float red[2 * kStatThreads / 64];
  const int64_t row = blockIdx.x;
  const T *z = draft + row * V;
  const T *y = teacher + row * V;
  const int tid = threadIdx.x;

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
    for (int64_t i = (int64_t)tid * 8; i < V; i += kStatThreads * 8) {
      float a[8], b[8];
      load8(z + i, a);
      load8(y + i, b);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float za = fmaf(sanitize(a[k]), kLog2e, -lz2);  // log2 q
        const float yb = fmaf(b[k], kLog2e, -ly2);            // log2 p
        const float e = __builtin_amdgcn_exp2f(fminf(za, yb));
        al += e;
        ss += za < yb ? e : 0.f;
      }
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
    alpha[row] = al;
    S_out[row] = ss;
    lse_q2[row] = lz2;
    lse_p2[row] = ly2;
  }
}

// One workgroup. c_s for every step; L in float64 with a fixed reduction order.
__global__ __launch_bounds__(1024) void e2etv_scan_kernel(const int32_t *__restrict__ step_off,
                                                         int32_t n_branches,
                                                         const float *__restrict__ alpha,
                                                         float w, float *__restrict__ coef,
                                                         float *__restrict__ loss) {
  __shared__ double red[1024 / 64];
  double part = 0.0;
  for (int b = threadIdx.x; b < n_branches; b += blockDim.x) {
    const int s0 = step_off[b], s1 = step_off[b + 1];
    // G_{W} = 1, G_i = 1 + alpha_{i+1} G_{i+1}; park G_i in coef
    double G = 1.0;
    for (int s = s1 - 1; s >= s0; --s) {
      coef[s] = (float)G;
      G = 1.0 + (double)alpha[s] * G;
    }
    // A_0 = 1, A_i = A_{i-1} alpha_i; c_i = -w A_{i-1} G_i; branch sum of A_j
    double A = 1.0, sumA = 0.0;
    for (int s = s0; s < s1; ++s) {
      const double Gi = coef[s];
      coef[s] = (float)(-(double)w * A * Gi);
      A *= (double)alpha[s];
      sumA += A;
    }
    part += sumA;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) t += red[k];
    loss[0] = (float)(1.0 - (double)w * t);
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kGradThreads) void e2etv_grad_kernel(
    const T *__restrict__ draft, const T *__restrict__ teacher, int64_t V,
    const float *__restrict__ lse_q2, const float *__restrict__ lse_p2,
    const float *__restrict__ S, const float *__restrict__ coef, float *__restrict__ grad,
    int32_t chunks_per_row) {
  const int64_t row = blockIdx.x / chunks_per_row;
  const int64_t chunk = blockIdx.x % chunks_per_row;
  const float lz2 = lse_q2[row], ly2 = lse_p2[row], c = coef[row], ss = S[row];
  const float cin = c * (1.f - ss), cout = -c * ss;  // coefficient inside / outside {q < p}
  const T *z = draft + row * V;
  const T *y = teacher + row * V;
  float *g = grad + row * V;
  if (VEC) {
    const int64_t i = (chunk * kGradThreads + threadIdx.x) * 8;
    if (i >= V) return;
    float a[8], b[8], r[8];
    load8(z + i, a);
    load8(y + i, b);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float za = fmaf(sanitize(a[k]), kLog2e, -lz2);
      const float yb = fmaf(b[k], kLog2e, -ly2);
      r[k] = (za < yb ? cin : cout) * __builtin_amdgcn_exp2f(za);
    }
    float4 *gp = reinterpret_cast<float4 *>(g + i);
    gp[0] = make_float4(r[0], r[1], r[2], r[3]);
    gp[1] = make_float4(r[4], r[5], r[6], r[7]);
  } else {
    const int64_t i0 = (chunk * kGradThreads + threadIdx.x) * 8;
    for (int64_t i = i0; i < i0 + 8 && i < V; ++i) {
      const float za = fmaf(sanitize(load1(z + i)), kLog2e, -lz2);
      const float yb = fmaf(load1(y + i), kLog2e, -ly2);
      g[i] = (za < yb ? cin : cout) * __builtin_amdgcn_exp2f(za);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused single-read kernel (bf16 logits, row groups of whole branches).
//
// A cooperative grid is cut into teams of `team` workgroups. A team takes one
// row group (<= 16 supervised steps made of whole branches) at a time; member j
// owns vocabulary slice j of every row in the group and keeps the draft and
// teacher values of that slice in registers for the whole round:
//   phase A  per row: slice max and sum of 2^(x log2 e - max log2 e) for z and y
//   barrier  members exchange their (max, sum) partials -> row log-sum-exps
//   phase B  per row: slice sums of 2^min(z', y') (alpha) and of 2^z' on {z' < y'} (S)
//   barrier  members exchange (alpha, S) partials -> per-branch scan -> c_s
//   phase C  gradient c_s q (1[z' < y'] - S) written straight from registers
// so every logit is read from HBM once and every gradient element written once.
// Partial buffers are double-buffered by round parity; the barrier is a
// monotonic per-team counter with a bounded spin that raises a status flag
// (the loss becomes NaN) instead of hanging. All combines run in a fixed order,
// so the results are bitwise reproducible.

constexpr int kFWaves = 4;                 // waves per workgroup
constexpr int kFSlots = 4;                 // rows per wave per round
constexpr int kFRows = kFWaves * kFSlots;  // rows per group
constexpr int kFThreads = kFWaves * 64;
constexpr int kFMaxGrid = 2048;
constexpr int kFMaxTeams = 512;
constexpr int kFCounterStride = 32;        // one 128-byte line per team counter
constexpr unsigned kFSpinLimit = 1u << 22;
constexpr int kFMaxTeam = 128;             // members per team the combine buffers allow
static_assert(kFRows == SPEC_ROW_GROUP, "row groups are planned for this kernel shape");

struct FusedArgs {
  const uint4 *z;          // draft rows, 8 bf16 per vector
  const uint4 *y;          // teacher rows
  int64_t V8;              // vectors per row
  const int32_t *group_off;
  int32_t n_groups;
  const int32_t *step_branch;
  const int32_t *step_off;
  int32_t team, n_teams;
  float w;
  float *alpha;
  float4 *grad;            // 2 float4 per vector
  float4 *lse_part;        // [n_teams][2][kFRows][team]
  float2 *as_part;         // [n_teams][2][kFRows][team]
  double *branch_sum;      // [B]
  unsigned *bar;           // [n_teams * kFCounterStride]
  unsigned *status;
  int want_grad;
};

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// bf16 NaN halves become -inf (inactive draft support).
__device__ inline uint32_t nan_to_neginf2(uint32_t w) {
  if ((w & 0x7fffu) > 0x7f80u) w = (w & 0xffff0000u) | 0xff80u;
  if (((w >> 16) & 0x7fffu) > 0x7f80u) w = (w & 0x0000ffffu) | 0xff800000u;
  return w;
}
__device__ inline float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Raw buffer access to one logit or gradient row: the row base sits in a
// wave-uniform descriptor, lanes carry one 32-bit offset and each vector of a
// lane adds an immediate, so the address math costs almost no VGPRs.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ inline uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 f) {
  u32x4 v;
  v.x = __float_as_uint(f.x);
  v.y = __float_as_uint(f.y);
  v.z = __float_as_uint(f.z);
  v.w = __float_as_uint(f.w);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

__device__ inline uint32_t comp(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Partials cross workgroups (and XCDs, whose L2s are not coherent with each
// other) through agent-scope atomic stores and loads, which go to the
// coherence point; no L2-wide writeback or invalidate is needed.
__device__ inline void st_agent(float *p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t ld_agent2(const float *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(reinterpret_cast<const uint64_t *>(p)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copy n 8-byte words of partials to LDS with coherent loads, four in flight per thread.
__device__ inline void fetch_partials(uint64_t *dst, const float *src, int n) {
  for (int base = threadIdx.x; base < n; base += 4 * kFThreads) {
    uint64_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = base + i * kFThreads;
      if (idx < n) v[i] = ld_agent2(src + 2 * idx);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = base + i * kFThreads;
      if (idx < n) dst[idx] = v[i];
    }
  }
}

// A member arrives at a barrier in two steps: bar_flush() waits until this
// workgroup's agent-scope partial stores have completed (so arrival implies
// visibility), bar_wait() bumps the team counter and spins until every member
// has arrived. Work issued between the two overlaps the wait. Barrier n of a
// team completes when its counter reaches team * n; a bounded spin raises a
// status flag instead of hanging.
__device__ inline void bar_flush() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}
__device__ inline bool bar_wait(unsigned *ctr, unsigned target, unsigned *status, int *s_ok) {
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    unsigned spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
          ++spins > kFSpinLimit) {
        __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
    }
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// Issue the loads of this member's slice of one array for rows [s0, s0 + nr)
// of a group. Nothing here waits for the data; vectors outside the slice are
// masked to -inf when the slice is first used (mask_slice).
template <int VPL>
__device__ inline void load_slice(uint4 (&dst)[kFSlots][VPL], const uint4 *base, int64_t V8,
                                  int s0, int nr, int wv, int lane, int64_t vb, int64_t ve) {
  const uint32_t row_bytes = (uint32_t)(V8 * 16);
  const uint32_t voff = (uint32_t)((vb + lane) * 16);
#pragma unroll
  for (int rs = 0; rs < kFSlots; ++rs) {
    const int r = rs * kFWaves + wv;
    const __amdgpu_buffer_rsrc_t rr = row_rsrc(base + (int64_t)(s0 + (r < nr ? r : 0)) * V8, row_bytes);
#pragma unroll
    for (int k = 0; k < VPL; ++k) dst[rs][k] = buf_load16(rr, voff + 1024u * k);
  }
}

template <int VPL>
__device__ inline void mask_slice(uint4 (&v)[kFSlots][VPL], int lane, int64_t vb, int64_t ve) {
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    if (vb + lane + 64 * k < ve) continue;
#pragma unroll
    for (int rs = 0; rs < kFSlots; ++rs)
      v[rs][k] = make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
  }
}

// Wave-level (max, sum 2^(x log2 e - max log2 e)) over one slot of a slice.
template <int VPL>
__device__ inline float2 slot_lse(const uint4 (&v)[VPL]) {
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = comp(v[k], i);
      m = fmaxf(m, fmaxf(lo_f(w), hi_f(w)));
    }
  m = wave_max(m);
  float sm = 0.f;
  if (m != -INFINITY) {
    const float nm = -m * kLog2e;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w = comp(v[k], i);
        asm volatile("" : "+v"(w));  // unpack again rather than keep the unpacked slot live
        sm += __builtin_amdgcn_exp2f(fmaf(lo_f(w), kLog2e, nm));
        sm += __builtin_amdgcn_exp2f(fmaf(hi_f(w), kLog2e, nm));
      }
  }
  return make_float2(m, wave_sum(sm));
}

template <int VPL>
__global__ __launch_bounds__(kFThreads) void e2etv_fused_kernel(FusedArgs a) {
  static_assert(VPL * 8 <= 32, "indicator bits of a slot fit one register");
  extern __shared__ float4 s_part[];           // [kFRows][team] partials of the current barrier
  __shared__ float s_lz[kFRows], s_ly[kFRows], s_al[kFRows], s_S[kFRows];
  __shared__ float s_cin[kFRows], s_cout[kFRows];
  __shared__ float s_myp[kFRows][2];           // this member's teacher partial per row
  __shared__ int s_ok;

  const int T = a.team;
  const int team = blockIdx.x / T;
  const int mem = blockIdx.x % T;
  if (team >= a.n_teams || team >= a.n_groups) return;  // uniform over the team
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int64_t vb = a.V8 * mem / T, ve = a.V8 * (mem + 1) / T;  // this member's vectors
  unsigned *ctr = a.bar + (size_t)team * kFCounterStride;
  unsigned nbar = 0;
  const uint32_t row_bytes = (uint32_t)(a.V8 * 16);
  const uint32_t voff = (uint32_t)((vb + lane) * 16);

  uint4 zr[kFSlots][VPL], yr[kFSlots][VPL];
  uint32_t bits[kFSlots];
  int g = team;
  int s0 = a.group_off[g], nr = a.group_off[g + 1] - s0;
  load_slice<VPL>(yr, a.y, a.V8, s0, nr, wv, lane, vb, ve);
  load_slice<VPL>(zr, a.z, a.V8, s0, nr, wv, lane, vb, ve);

  for (int round = 0;; ++round) {
    const int par = round & 1;
    float4 *lse_part = a.lse_part + ((size_t)(team * 2 + par) * kFRows) * T;
    float2 *as_part = a.as_part + ((size_t)(team * 2 + par) * kFRows) * T;

    // ---------------- phase A: teacher partials first (its slice arrived earlier), then draft
    mask_slice<VPL>(yr, lane, vb, ve);
#pragma unroll
    for (int rs = 0; rs < kFSlots; ++rs) {
      const int r = rs * kFWaves + wv;
      if (r >= nr) continue;  // wave-uniform
      const float2 py = slot_lse<VPL>(yr[rs]);
      if (lane == 0) {
        s_myp[r][0] = py.x;
        s_myp[r][1] = py.y;
      }
    }
    mask_slice<VPL>(zr, lane, vb, ve);
#pragma unroll
    for (int rs = 0; rs < kFSlots; ++rs) {
      const int r = rs * kFWaves + wv;
      if (r >= nr) continue;
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        zr[rs][k].x = nan_to_neginf2(zr[rs][k].x);
        zr[rs][k].y = nan_to_neginf2(zr[rs][k].y);
        zr[rs][k].z = nan_to_neginf2(zr[rs][k].z);
        zr[rs][k].w = nan_to_neginf2(zr[rs][k].w);
      }
      const float2 pz = slot_lse<VPL>(zr[rs]);
      if (lane == 0) {
        float *dst = reinterpret_cast<float *>(lse_part + (size_t)r * T + mem);
        st_agent(dst, pz.x);
        st_agent(dst + 1, pz.y);
        st_agent(dst + 2, s_myp[r][0]);
        st_agent(dst + 3, s_myp[r][1]);
      }
    }
    bar_flush();
    if (!bar_wait(ctr, (unsigned)T * ++nbar, a.status, &s_ok)) return;

    // ---------------- combine: row log-sum-exps (fixed order over members)
    fetch_partials(reinterpret_cast<uint64_t *>(s_part), reinterpret_cast<const float *>(lse_part),
                   nr * T * 2);
    __syncthreads();
    {
      const int p = tid >> 3, sub = tid & 7;  // 32 (row, array) pairs x 8 lanes
      const int r = p >> 1, arr = p & 1;
      float m = -INFINITY, sm = 0.f;
      if (r < nr)
        for (int j = sub; j < T; j += 8) {
          const float4 e = s_part[r * T + j];
          lse_merge(m, sm, arr ? e.z : e.x, arr ? e.w : e.y);
        }
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {
        const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(sm, off);
        lse_merge(m, sm, m2, s2);
      }
      if (sub == 0 && r < nr) (arr ? s_ly : s_lz)[r] = m * kLog2e + log2f(sm);
    }
    __syncthreads();

    // ---------------- phase B: alpha and S partials, and the indicator bits of z' < y'
#pragma unroll
    for (int rs = 0; rs < kFSlots; ++rs) {
      const int r = rs * kFWaves + wv;
      bits[rs] = 0u;
      if (r >= nr) continue;
      const float lz = s_lz[r], ly = s_ly[r];
      float al = 0.f, ss = 0.f;
      uint32_t bm = 0u;
#pragma unroll
      for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t wz = comp(zr[rs][k], i), wy = comp(yr[rs][k], i);
          asm volatile("" : "+v"(wz), "+v"(wy));
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float za = fmaf(h ? hi_f(wz) : lo_f(wz), kLog2e, -lz);
            const float yb = fmaf(h ? hi_f(wy) : lo_f(wy), kLog2e, -ly);
            const float e = __builtin_amdgcn_exp2f(fminf(za, yb));
            const bool in = za < yb;
            al += e;
            ss += in ? e : 0.f;
            bm |= (uint32_t)in << (8 * k + 2 * i + h);
          }
        }
      bits[rs] = bm;
      al = wave_sum(al);
      ss = wave_sum(ss);
      if (lane == 0) {
        float *dst = reinterpret_cast<float *>(as_part + (size_t)r * T + mem);
        st_agent(dst, al);
        st_agent(dst + 1, ss);
      }
    }
    bar_flush();
    // the teacher slice is dead now: fetch the next group's while the team syncs
    const int gn = g + a.n_teams;
    const bool has_next = gn < a.n_groups;
    int s0n = 0, nrn = 0;
    if (has_next) {
      s0n = a.group_off[gn];
      nrn = a.group_off[gn + 1] - s0n;
      load_slice<VPL>(yr, a.y, a.V8, s0n, nrn, wv, lane, vb, ve);
    }
    if (!bar_wait(ctr, (unsigned)T * ++nbar, a.status, &s_ok)) return;

    // ---------------- combine alpha and S, then the per-branch coefficients
    float2 *s_part2 = reinterpret_cast<float2 *>(s_part);
    fetch_partials(reinterpret_cast<uint64_t *>(s_part2), reinterpret_cast<const float *>(as_part),
                   nr * T);
    __syncthreads();
    {
      const int r = tid >> 4, sub = tid & 15;  // 16 rows x 16 lanes
      float al = 0.f, ss = 0.f;
      if (r < nr)
        for (int j = sub; j < T; j += 16) {
          const float2 e = s_part2[r * T + j];
          al += e.x;
          ss += e.y;
        }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        al += __shfl_xor(al, off);
        ss += __shfl_xor(ss, off);
      }
      if (sub == 0 && r < nr) {
        s_al[r] = al;
        s_S[r] = ss;
      }
    }
    __syncthreads();
    if (tid < nr) {
      const int s = s0 + tid;
      const int b = a.step_branch[s];
      const int bs0 = a.step_off[b], bs1 = a.step_off[b + 1];
      double A = 1.0;  // A_{i-1}
      for (int j = bs0; j < s; ++j) A *= (double)s_al[j - s0];
      double G = 1.0;  // G_i
      for (int j = bs1 - 1; j > s; --j) G = 1.0 + (double)s_al[j - s0] * G;
      const double c = -(double)a.w * A * G;
      const double S = (double)s_S[tid];
      s_cin[tid] = (float)(c * (1.0 - S));
      s_cout[tid] = (float)(-c * S);
      if (mem == 0) {
        a.alpha[s] = s_al[tid];
        if (s == bs0) {
          double P = 1.0, sum = 0.0;
          for (int j = bs0; j < bs1; ++j) {
            P *= (double)s_al[j - s0];
            sum += P;
          }
          a.branch_sum[b] = sum;
        }
      }
    }
    __syncthreads();

    // ---------------- phase C: gradient from the draft slice and the indicator bits
    if (a.want_grad) {
#pragma unroll
      for (int rs = 0; rs < kFSlots; ++rs) {
        const int r = rs * kFWaves + wv;
        if (r >= nr) continue;
        const float lz = s_lz[r], cin = s_cin[r], cout = s_cout[r];
        const uint32_t bm = bits[rs];
        const __amdgpu_buffer_rsrc_t rg = row_rsrc(a.grad + (int64_t)(s0 + r) * a.V8 * 2, 2 * row_bytes);
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          if (vb + lane + 64 * k >= ve) continue;
          float gv[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t wz = comp(zr[rs][k], i);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float za = fmaf(h ? hi_f(wz) : lo_f(wz), kLog2e, -lz);
              const bool in = (bm >> (8 * k + 2 * i + h)) & 1u;
              gv[2 * i + h] = (in ? cin : cout) * __builtin_amdgcn_exp2f(za);
            }
          }
          buf_store16(rg, 2 * voff + 2048u * k, make_float4(gv[0], gv[1], gv[2], gv[3]));
          buf_store16(rg, 2 * voff + 2048u * k + 16u, make_float4(gv[4], gv[5], gv[6], gv[7]));
        }
      }
    }
    if (!has_next) break;
    g = gn;
    s0 = s0n;
    nr = nrn;
    load_slice<VPL>(zr, a.z, a.V8, s0, nr, wv, lane, vb, ve);
  }
}

__global__ void e2etv_fused_reset(unsigned *bar, int n, unsigned *status) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) bar[i] = 0u;
  if (threadIdx.x == 0) *status = 0u;
}

// L = 1 - w * sum_b branch_sum[b], float64, fixed order; NaN if a barrier timed out.
__global__ __launch_bounds__(1024) void e2etv_fused_loss(const double *__restrict__ branch_sum,
                                                        int32_t n_branches, float w,
                                                        const unsigned *status, float *loss) {
  __shared__ double red[1024 / 64];
  double part = 0.0;
  for (int b = threadIdx.x; b < n_branches; b += blockDim.x) part += branch_sum[b];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) t += red[k];
    loss[0] = *status ? NAN : (float)(1.0 - (double)w * t);
  }
}

namespace {

template <typename T, bool VEC>
hipError_t launch_typed(const spec_tree_layout &L, int64_t V, const void *draft,
                        const void *teacher, float w, float *alpha, float *loss, float *grad,
                        const E2etvWork &ws, hipStream_t s) {
  const T *z = static_cast<const T *>(draft);
  const T *y = static_cast<const T *>(teacher);
  const int64_t R = L.n_steps;
  hipLaunchKernelGGL((e2etv_stats_kernel<T, VEC>), dim3((unsigned)R), dim3(kStatThreads), 0, s, z,
                     y, V, alpha, ws.S, ws.lse_q2, ws.lse_p2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_stats");
  hipLaunchKernelGGL(e2etv_scan_kernel, dim3(1), dim3(1024), 0, s, L.step_off, L.n_branches,
                     alpha, w, ws.coef, loss);
  e = hipGetLastError();
  if (e != hipSuccess || !grad) return e;
  prof_mark(s, "e2etv_scan");
  const int64_t per_block = (int64_t)kGradThreads * 8;
  const int64_t chunks = (V + per_block - 1) / per_block;
  if (chunks * R > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((e2etv_grad_kernel<T, VEC>), dim3((unsigned)(chunks * R)), dim3(kGradThreads),
                     0, s, z, y, V, ws.lse_q2, ws.lse_p2, ws.S, ws.coef, grad, (int32_t)chunks);
  e = hipGetLastError();
  prof_mark(s, "e2etv_grad");
  return e;
}

struct FusedDevice {
  int cus = 0, coop = 0, occ4 = -1;
};

// Device properties and the fused kernel's occupancy, looked up once per device.
FusedDevice fused_device(int dev, size_t lds) {
  static std::mutex mu;
  static FusedDevice cache[64];
  static size_t cache_lds[64];
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= 64) return FusedDevice{};
  FusedDevice &d = cache[dev];
  if (d.cus == 0) {
    hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    hipDeviceGetAttribute(&d.coop, hipDeviceAttributeCooperativeLaunch, dev);
  }
  if (d.occ4 < 0 || cache_lds[dev] != lds) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)e2etv_fused_kernel<4>,
                                                     kFThreads, lds) != hipSuccess)
      n = 0;
    d.occ4 = n;
    cache_lds[dev] = lds;
  }
  return d;
}

// Launch the fused path if the problem fits it; *used says whether it ran.
hipError_t launch_fused(const spec_tree_layout &L, int64_t V, const void *draft, const void *teacher,
                        float w, float *alpha, float *loss, float *grad, const E2etvWork &ws,
                        hipStream_t s, bool *used) {
  *used = false;
  constexpr int VPL = 4;
  const int64_t V8 = V / 8;
  const int64_t T = (V8 + 64 * VPL - 1) / (64 * VPL);
  if (L.max_branch_len > kFRows || L.n_row_groups < 1 || T > kFMaxTeam) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)kFRows * T * sizeof(float4);
  const FusedDevice d = fused_device(dev, lds);
  if (!d.coop || d.occ4 < 1 || d.cus < 1) return hipSuccess;
  int64_t n_teams = std::min<int64_t>((int64_t)d.occ4 * d.cus, kFMaxGrid) / T;
  n_teams = std::min<int64_t>({n_teams, (int64_t)L.n_row_groups, (int64_t)kFMaxTeams});
  if (n_teams < 1) return hipSuccess;

  hipLaunchKernelGGL(e2etv_fused_reset, dim3(1), dim3(256), 0, s, ws.bar,
                     (int)(n_teams * kFCounterStride), ws.status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  FusedArgs a;
  a.z = static_cast<const uint4 *>(draft);
  a.y = static_cast<const uint4 *>(teacher);
  a.V8 = V8;
  a.group_off = L.row_group_off;
  a.n_groups = L.n_row_groups;
  a.step_branch = L.step_branch;
  a.step_off = L.step_off;
  a.team = (int32_t)T;
  a.n_teams = (int32_t)n_teams;
  a.w = w;
  a.alpha = alpha;
  a.grad = reinterpret_cast<float4 *>(grad);
  a.lse_part = ws.lse_part;
  a.as_part = ws.as_part;
  a.branch_sum = ws.branch_sum;
  a.bar = ws.bar;
  a.status = ws.status;
  a.want_grad = grad != nullptr;
  void *args[] = {&a};
  e = hipLaunchCooperativeKernel((const void *)e2etv_fused_kernel<VPL>, dim3((unsigned)(n_teams * T)),
                                 dim3(kFThreads), args, (unsigned)lds, s);
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_fused");
  hipLaunchKernelGGL(e2etv_fused_loss, dim3(1), dim3(1024), 0, s, ws.branch_sum, L.n_branches, w,
                     ws.status, loss);
  e = hipGetLastError();
  if (e == hipSuccess) prof_mark(s, "e2etv_loss");
  *used = true;
  return e;
}

}  // namespace

hipError_t launch_e2etv(const spec_tree_layout &L, int64_t V, spec_dtype dtype, const void *draft,
                        const void *teacher, float w, float *alpha, float *loss, float *grad,
                        const E2etvWork &ws, hipStream_t s) {
  const bool vec = (V % 8) == 0;
  if (dtype == SPEC_BF16 && vec) {
    bool used = false;
    hipError_t e = launch_fused(L, V, draft, teacher, w, alpha, loss, grad, ws, s, &used);
    if (e != hipSuccess || used) return e;
  }
  if (dtype == SPEC_BF16)
    return vec ? launch_typed<__bf16, true>(L, V, draft, teacher, w, alpha, loss, grad, ws, s)
               : launch_typed<__bf16, false>(L, V, draft, teacher, w, alpha, loss, grad, ws, s);
  return vec ? launch_typed<float, true>(L, V, draft, teacher, w, alpha, loss, grad, ws, s)
             : launch_typed<float, false>(L, V, draft, teacher, w, alpha, loss, grad, ws, s);
}

}  // namespace spec
