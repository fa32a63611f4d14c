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

// Tiled K and V for the bf16 head-dim-128 attention kernel, which copies whole
// 64-key tiles into LDS with direct-to-LDS loads (no registers, no shuffles on
// the way). Per KV head g and key tile t (keys 64t .. 64t+63, zero past N):
//   Kt[g][t]: 64 rows x 16 chunks of 8 dims, rotated like rope_k; chunk c of row r
//             sits in slot r*16 + (c ^ (r & 15)), so the 32 rows an MFMA fragment
//             reads fall in distinct LDS banks;
//   Vt[g][t]: V transposed, 128 dims x 8 chunks of 8 keys; within each 16-key
//             group the key quads are stored in the order [0, 2, 1, 3] (the order
//             the P^T operand of the P V MFMA expects), and chunk c of dim d sits
//             in slot d*8 + (c ^ vt_swizzle(d)).
// One 256-thread workgroup per (tile, head); V goes through LDS for the transpose.
constexpr int kTileKeys = kKeyTile;

__global__ __launch_bounds__(256) void kv_tile_kernel(const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
                                                      __bf16 *__restrict__ kt, __bf16 *__restrict__ vt,
                                                      const float2 *__restrict__ tab,
                                                      const int32_t *__restrict__ row_pos, int64_t n_rows,
                                                      int32_t hkv, int32_t n_tiles) {
  constexpr int D = 128, H = 64, CH = 16;
  __shared__ __bf16 vs[kTileKeys][D + 8];
  const int tile = blockIdx.x % n_tiles, g = blockIdx.x / n_tiles;
  const int tid = threadIdx.x;
  const int64_t key0 = (int64_t)tile * kTileKeys;
  // V rows of the tile into LDS (zero past the last row)
  for (int i = tid; i < kTileKeys * CH; i += 256) {
    const int r = i / CH, c = i % CH;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (key0 + r < n_rows) x = *reinterpret_cast<const uint4 *>(v + ((key0 + r) * hkv + g) * D + c * 8);
    *reinterpret_cast<uint2 *>(&vs[r][c * 8]) = make_uint2(x.x, x.y);
    *reinterpret_cast<uint2 *>(&vs[r][c * 8 + 4]) = make_uint2(x.z, x.w);
  }
  // K: rotate and store swizzled chunks
  __bf16 *kdst = kt + ((int64_t)g * n_tiles + tile) * kTileKeys * D;
  for (int p = tid; p < kTileKeys * CH; p += 256) {
    const int r = p / CH, c = (p % CH) ^ (r & (CH - 1));
    __bf16 y[8];
    if (key0 + r < n_rows) {
      const __bf16 *src = k + ((key0 + r) * hkv + g) * D;
      const int j0 = (c % (CH / 2)) * 8;  // pair index of the chunk's first dim
      const float2 *cs = tab + (int64_t)row_pos[key0 + r] * H + j0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x1 = (float)src[j0 + e], x2 = (float)src[j0 + e + H];
        const float2 t = cs[e];
        y[e] = c < CH / 2 ? (__bf16)(x1 * t.x - x2 * t.y) : (__bf16)(x2 * t.x + x1 * t.y);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (__bf16)0.f;
    }
    uint4 pk;
    __builtin_memcpy(&pk, y, 16);
    *reinterpret_cast<uint4 *>(kdst + (int64_t)p * 8) = pk;
  }
  __syncthreads();
  // V^T: slot p = d*8 + c' holds logical chunk c = c' ^ vt_swizzle(d): positions
  // 8c .. 8c+7 of dim d, i.e. key quads [0, 2, 1, 3][2 (c & 1) + 0, 1] of the
  // 16-key group c / 2
  __bf16 *vdst = vt + ((int64_t)g * n_tiles + tile) * kTileKeys * D;
  for (int p = tid; p < D * 8; p += 256) {
    const int d = p / 8, c = (p % 8) ^ vt_swizzle(d);
    const int grp = c / 2, q0 = (c & 1) ? 1 : 0;  // quads 0, 2 (c even) or 1, 3 (c odd)
    __bf16 y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = vs[16 * grp + 4 * q0 + e][d];
      y[4 + e] = vs[16 * grp + 4 * (q0 + 2) + e][d];
    }
    uint4 pk;
    __builtin_memcpy(&pk, y, 16);
    *reinterpret_cast<uint4 *>(vdst + (int64_t)p * 8) = pk;
  }
}

hipError_t launch_kv_tiles(const void *k, const void *v, void *kt, void *vt, const float2 *tab,
                           const int32_t *row_pos, int64_t n_rows, int32_t hkv, hipStream_t stream) {
  const int64_t n_tiles = (n_rows + kTileKeys - 1) / kTileKeys;
  if (n_tiles * hkv > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_tile_kernel, dim3((unsigned)(n_tiles * hkv)), dim3(256), 0, stream,
                     static_cast<const __bf16 *>(k), static_cast<const __bf16 *>(v),
                     static_cast<__bf16 *>(kt), static_cast<__bf16 *>(vt), tab, row_pos, n_rows, hkv,
                     (int32_t)n_tiles);
  return hipGetLastError();
}

}  // namespace spec
