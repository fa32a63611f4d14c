// RoPE at semantic positions ([SpecOPD notes page, "Equations"]: a branch token
// y_{b,i} sits at position a_b + i, not at its packed offset).
//
// Rotate-half form: dimension j pairs with j + D/2 and turns by the angle
// pos * base^(-2j/D). A table of (cos, sin) per (position, j) is built once per
// call with float64 angles (positions reach 32k, where a float32 product
// pos * theta would already be off by ~1e-3 rad), then K is rotated once into
// a head-major workspace [Hkv][N][D] that the attention kernel streams.
#include "common.h"

namespace spec {

__global__ void rope_table_kernel(float2 *__restrict__ tab, int32_t n_pos, int32_t half,
                                  double log_base) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_pos * half) return;
  const int pos = (int)(idx / half);
  const int j = (int)(idx % half);
  const double inv_freq = exp(-(double)(2 * j) / (double)(2 * half) * log_base);
  double s, c;
  sincos((double)pos * inv_freq, &s, &c);
  tab[idx] = make_float2((float)c, (float)s);
}

hipError_t launch_rope_table(float2 *tab, int32_t n_pos, int32_t half, double base,
                             hipStream_t stream) {
  const int64_t n = (int64_t)n_pos * half;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     tab, n_pos, half, log(base));
  return hipGetLastError();
}

template <typename T>
__device__ inline float to_f32(T x);
template <>
__device__ inline float to_f32<float>(float x) { return x; }
template <>
__device__ inline float to_f32<__bf16>(__bf16 x) { return (float)x; }

template <typename T>
__device__ inline T from_f32(float x);
template <>
__device__ inline float from_f32<float>(float x) { return x; }
template <>
__device__ inline __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }  // round to nearest even

// One thread per (row, kv head, pair j). Reads k[r][g][j], k[r][g][j + D/2];
// writes the rotated pair to kws[g][r][.].
template <typename T>
__global__ void rope_k_kernel(const T *__restrict__ k, T *__restrict__ kws,
                              const float2 *__restrict__ tab, const int32_t *__restrict__ row_pos,
                              int64_t n_rows, int32_t hkv, int32_t half) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = n_rows * hkv * half;
  if (idx >= total) return;
  const int j = (int)(idx % half);
  const int64_t rg = idx / half;
  const int g = (int)(rg % hkv);
  const int64_t r = rg / hkv;
  const int D = 2 * half;
  const T *src = k + rg * D;
  const float x1 = to_f32(src[j]), x2 = to_f32(src[j + half]);
  const float2 cs = tab[(int64_t)row_pos[r] * half + j];
  T *dst = kws + ((int64_t)g * n_rows + r) * D;
  dst[j] = from_f32<T>(x1 * cs.x - x2 * cs.y);
  dst[j + half] = from_f32<T>(x2 * cs.x + x1 * cs.y);
}

hipError_t launch_rope_k(const void *k, void *kws, const float2 *tab, const int32_t *row_pos,
                         int64_t n_rows, int32_t hkv, int32_t D, spec_dtype dtype,
                         hipStream_t stream) {
  const int64_t n = n_rows * hkv * (D / 2);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(rope_k_kernel<__bf16>, grid, dim3(256), 0, stream,
                       static_cast<const __bf16 *>(k), static_cast<__bf16 *>(kws), tab, row_pos,
                       n_rows, hkv, D / 2);
  else
    hipLaunchKernelGGL(rope_k_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float *>(k), static_cast<float *>(kws), tab, row_pos,
                       n_rows, hkv, D / 2);
  return hipGetLastError();
}

}  // namespace spec
