// E2E-TV surrogate, loss and gradient with respect to the draft logits.
//
// [SpecOPD notes page, "Equations"]: alpha_{b,i} = sum_v min(q_v, p_v) over the
// full vocabulary; L = 1 - (1/(BW)) sum_b sum_j prod_{i<=j} alpha_{b,i}; samples
// and the teacher are fixed when differentiating; teacher mass outside the draft
// support is kept. [SpecOPD notes page, "Inputs and code mapping"]: low
// precision is promoted to float32; NaN draft entries are inactive support.
//
// Three kernels on the caller's stream:
//   e2etv_stats  a persistent grid, one 1024-thread workgroup per CU, walks the
//                rows; per row, pass 1 streams it for both log-sum-exps (online
//                max/sum per lane) and pass 2 re-streams it (partly from cache,
//                since only one row per CU is in flight) for
//                alpha = sum 2^min(z', y') and S = sum over {z' < y'} of 2^z', where
//                z' = z*log2(e) - lse2(z) is log2 q (and y' likewise log2 p);
//   e2etv_scan   one workgroup: per branch the suffix sums G and prefix products
//                A give c_s = dL/d alpha_s = -w A_{i-1} G_i (no division), and the
//                loss is reduced in float64 in a fixed order;
//   e2etv_grad   grad[s,u] = c_s * q_u * (1[z'_u < y'_u] - S_s), written once. The
//                statistics pass stores the decision z'_u < y'_u as a bitmask, so
//                the gradient reads the draft row and 1 bit per element, not the
//                teacher row (6.1 instead of 8 bytes per element).
// Every reduction has a fixed order, so results are bitwise reproducible. The
// strict test z' < y' is the same expression in all three places, so the set
// {q < p} used for S and for the gradient is the same set.
#include <algorithm>

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
    float *__restrict__ alpha, float *__restrict__ S_out, float *__restrict__ lse_q2,
    float *__restrict__ lse_p2, uint8_t *__restrict__ bits, int64_t bits_row) {
  __shared__ float red[2 * kStatThreads / 64];
  const int tid = threadIdx.x;
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
    alpha[row] = al;
    S_out[row] = ss;
    lse_q2[row] = lz2;
    lse_p2[row] = ly2;
  }
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

template <typename T, bool VEC>
hipError_t launch_typed(const spec_tree_layout &L, int64_t V, const void *draft,
                        const void *teacher, float w, float *alpha, float *loss, float *grad,
                        const E2etvWork &ws, hipStream_t s) {
  const T *z = static_cast<const T *>(draft);
  const T *y = static_cast<const T *>(teacher);
  const int64_t R = L.n_steps;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(R, cus));
  hipLaunchKernelGGL((e2etv_stats_kernel<T, VEC>), dim3((unsigned)grid), dim3(kStatThreads), 0, s, z,
                     y, R, V, alpha, ws.S, ws.lse_q2, ws.lse_p2, ws.bits, ws.bits_row);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_stats");
  hipLaunchKernelGGL(e2etv_scan_kernel, dim3(1), dim3(1024), 0, s, L.step_off, L.n_branches,
                     alpha, w, ws.coef, loss);
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

}  // namespace spec
