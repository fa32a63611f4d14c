// Ceiling probes for the roofline figures (measurement only; libspec_probe.so,
// loaded by the benchmark's ceiling mode, never by the scoring path).
//
// Each probe moves or computes a known amount and nothing else, so its launch
// duration gives the rate a tuned kernel of the same shape can reach on this chip:
//   spec_probe_read   read-only stream of 16-byte loads
//   spec_probe_write  write-only stream of 16-byte stores
//   spec_probe_mixed  two bf16 inputs read and one float32 output written per
//                     element (4 bytes read : 4 bytes written, the mix of the
//                     E2E-TV forward and backward over bf16 logits)
//   spec_probe_mfma   chains of v_mfma_f32_32x32x16_bf16 on register operands
//   spec_probe_mfma_lds the same MFMAs with a fresh 1 KB A fragment read from LDS
//                     every `reuse` of them (reuse 1 is the tree attention's
//                     dataflow: each K or V^T fragment feeds one MFMA); reuse 0
//                     only reads, for the LDS read rate
// Loads and stores can be marked non-temporal (the nt cache policy).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ inline uint4 ld16(const uint4 *p) {
  const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
  const u32x4 v = NT ? __builtin_nontemporal_load(q) : *q;
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool NT>
__device__ inline void st16(uint4 *p, uint4 v) {
  u32x4 *q = reinterpret_cast<u32x4 *>(p);
  const u32x4 w = {v.x, v.y, v.z, v.w};
  if constexpr (NT)
    __builtin_nontemporal_store(w, q);
  else
    *q = w;
}

// The XOR of everything read is written only if it equals a value it never takes
// for the probe's inputs, so the loads cannot be dropped.
template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const uint4 *__restrict__ a, int64_t n16,
                                                              uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 u0 = ld16<NT>(a + i), u1 = ld16<NT>(a + i + stride);
    const uint4 u2 = ld16<NT>(a + i + 2 * stride), u3 = ld16<NT>(a + i + 3 * stride);
    acc ^= u0.x ^ u0.y ^ u0.z ^ u0.w ^ u1.x ^ u1.y ^ u1.z ^ u1.w;
    acc ^= u2.x ^ u2.y ^ u2.z ^ u2.w ^ u3.x ^ u3.y ^ u3.z ^ u3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 u = ld16<NT>(a + i);
    acc ^= u.x ^ u.y ^ u.z ^ u.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void probe_write_kernel(uint4 *__restrict__ out, int64_t n16, uint32_t v) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const uint4 w = make_uint4(v, v, v, v);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) st16<NT>(out + i, w);
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline void diff8(uint4 x, uint4 y, uint4 &o0, uint4 &o1) {
  o0 = make_uint4(__float_as_uint(bf_lo(x.x) - bf_lo(y.x)), __float_as_uint(bf_hi(x.x) - bf_hi(y.x)),
                  __float_as_uint(bf_lo(x.y) - bf_lo(y.y)), __float_as_uint(bf_hi(x.y) - bf_hi(y.y)));
  o1 = make_uint4(__float_as_uint(bf_lo(x.z) - bf_lo(y.z)), __float_as_uint(bf_hi(x.z) - bf_hi(y.z)),
                  __float_as_uint(bf_lo(x.w) - bf_lo(y.w)), __float_as_uint(bf_hi(x.w) - bf_hi(y.w)));
}

// out[e] = a[e] - b[e] for 8 elements per thread and step (32 bytes read, 32
// written), UNROLL steps' loads issued before their stores.
template <bool NTL, bool NTS, int UNROLL>
__global__ __launch_bounds__(kThreads) void probe_mixed_kernel(const uint4 *__restrict__ a,
                                                               const uint4 *__restrict__ b,
                                                               uint4 *__restrict__ out, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (UNROLL - 1) * stride < n8; i += UNROLL * stride) {
    uint4 x[UNROLL], y[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      x[u] = ld16<NTL>(a + i + u * stride);
      y[u] = ld16<NTL>(b + i + u * stride);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      uint4 o0, o1;
      diff8(x[u], y[u], o0, o1);
      st16<NTS>(out + 2 * (i + u * stride), o0);
      st16<NTS>(out + 2 * (i + u * stride) + 1, o1);
    }
  }
  for (; i < n8; i += stride) {
    uint4 o0, o1;
    diff8(ld16<NTL>(a + i), ld16<NTL>(b + i), o0, o1);
    st16<NTS>(out + 2 * i, o0);
    st16<NTS>(out + 2 * i + 1, o1);
  }
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// Four independent accumulator chains per wave; operands stay in registers.
__global__ __launch_bounds__(kThreads) void probe_mfma_kernel(float *__restrict__ out, int iters) {
  bf16x8 a, b;
  const float s = (float)(threadIdx.x & 7) * 0.125f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(s + j);
    b[j] = (__bf16)(s - j);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) t += c0[j] + c1[j] + c2[j] + c3[j];
  if (t == 1.2345f) out[blockIdx.x] = t;
}

// A 32 KB LDS buffer of 32 fragments (1 KB each, lane l holding bytes 16l..16l+15:
// a conflict-free ds_read_b128); a wave reads 8 of them per iteration, the next
// iteration's 8 issued before this one's are used.
template <int REUSE>
__global__ __launch_bounds__(kThreads) void probe_mfma_lds_kernel(float *__restrict__ out, int iters) {
  constexpr int NF = 32;
  __shared__ u32x4 buf[NF * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < NF * 64; i += kThreads) {
    const uint32_t v = 0x3f803f80u ^ ((uint32_t)i & 0x00070007u);  // bf16 values near 1
    buf[i] = u32x4{v, v, v, v};
  }
  __syncthreads();
  bf16x8 b;
  const float sb = (float)(lane & 7) * 0.125f;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = (__bf16)(sb - j);
  f32x16 c[4] = {};
  u32x4 fa[8], fb[8];
  auto rd = [&](int it, u32x4 (&f)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = buf[((it * 8 + j) & (NF - 1)) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
  };
  auto use = [&](const u32x4 (&f)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (REUSE == 0) {
        asm volatile("" ::"v"(f[j]));
      } else {
        const bf16x8 a = __builtin_bit_cast(bf16x8, f[j]);
#pragma unroll
        for (int r = 0; r < REUSE; ++r)
          c[(j * REUSE + r) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[(j * REUSE + r) & 3], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  rd(0, fa);
  for (int it = 0; it < iters; it += 2) {
    rd(it + 1, fb);
    use(fa);
    rd(it + 2, fa);
    use(fb);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) t += c[0][j] + c[1][j] + c[2][j] + c[3][j];
  if (t == 1.2345f) out[blockIdx.x] = t;
}

int grid_for(int64_t n, int cap) {
  const int64_t g = (n + kThreads - 1) / kThreads;
  return (int)(g < cap ? (g < 1 ? 1 : g) : cap);
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from a. Returns a hipError_t.
int spec_probe_read(const void *a, int64_t bytes, void *sink, int nontemporal, int grid, void *stream) {
  const int64_t n16 = bytes / 16;
  const int g = grid > 0 ? grid : grid_for(n16 / 4, 1 << 20);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(probe_read_kernel<true>, dim3(g), dim3(kThreads), 0, s, (const uint4 *)a, n16, (uint32_t *)sink);
  else
    hipLaunchKernelGGL(probe_read_kernel<false>, dim3(g), dim3(kThreads), 0, s, (const uint4 *)a, n16, (uint32_t *)sink);
  return (int)hipGetLastError();
}

// Write `bytes` (a multiple of 16) to out.
int spec_probe_write(void *out, int64_t bytes, int nontemporal, int grid, void *stream) {
  const int64_t n16 = bytes / 16;
  const int g = grid > 0 ? grid : grid_for(n16, 1 << 20);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(probe_write_kernel<true>, dim3(g), dim3(kThreads), 0, s, (uint4 *)out, n16, 0u);
  else
    hipLaunchKernelGGL(probe_write_kernel<false>, dim3(g), dim3(kThreads), 0, s, (uint4 *)out, n16, 0u);
  return (int)hipGetLastError();
}

// out[e] = a[e] - b[e] over n elements (a multiple of 8): bf16 a, b; float32 out.
// unroll 1 or 4: octets per thread whose loads are in flight together.
int spec_probe_mixed(const void *a, const void *b, void *out, int64_t n, int nt_load, int nt_store, int unroll,
                     int grid, void *stream) {
  const int64_t n8 = n / 8;
  const int u = unroll == 4 ? 4 : 1;
  const int g = grid > 0 ? grid : grid_for(n8 / u, 1 << 20);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4 *pa = (const uint4 *)a, *pb = (const uint4 *)b;
  uint4 *po = (uint4 *)out;
  const int sel = (nt_load ? 1 : 0) | (nt_store ? 2 : 0) | (u == 4 ? 4 : 0);
  switch (sel) {
    case 0: hipLaunchKernelGGL((probe_mixed_kernel<false, false, 1>), dim3(g), dim3(kThreads), 0, s, pa, pb, po, n8); break;
    case 1: hipLaunchKernelGGL((probe_mixed_kernel<true, false, 1>), dim3(g), dim3(kThreads), 0, s, pa, pb, po, n8); break;
    case 2: hipLaunchKernelGGL((probe_mixed_kernel<false, true, 1>), dim3(g), dim3(kThreads), 0, s, pa, pb, po, n8); break;
    case 3: hipLaunchKernelGGL((probe_mixed_kernel<true, true, 1>), dim3(g), dim3(kThreads), 0, s, pa, pb, po, n8); break;
    case 4: hipLaunchKernelGGL((probe_mixed_kernel<false, false, 4>), dim3(g), dim3(kThreads), 0, s, pa, pb, po, n8); break;
    case 5: hipLaunchKernelGGL((probe_mixed_kernel<true, false, 4>), dim3(g), dim3(kThreads), 0, s, pa, pb, po, n8); break;
    case 6: hipLaunchKernelGGL((probe_mixed_kernel<false, true, 4>), dim3(g), dim3(kThreads), 0, s, pa, pb, po, n8); break;
    default: hipLaunchKernelGGL((probe_mixed_kernel<true, true, 4>), dim3(g), dim3(kThreads), 0, s, pa, pb, po, n8); break;
  }
  return (int)hipGetLastError();
}

// `blocks` workgroups of 4 waves, each wave 4 * iters MFMAs of 32x32x16
// (32768 flops each). out needs `blocks` floats.
int spec_probe_mfma(void *out, int blocks, int iters, void *stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     (float *)out, iters);
  return (int)hipGetLastError();
}

// `blocks` workgroups of 4 waves; each wave reads 8 * iters 1 KB LDS fragments
// (iters even) and runs `reuse` MFMAs of 32x32x16 on each (reuse 0, 1, 2 or 4).
int spec_probe_mfma_lds(void *out, int blocks, int iters, int reuse, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  float *o = (float *)out;
  if (iters < 2 || (iters & 1)) return (int)hipErrorInvalidValue;
  switch (reuse) {
    case 0: hipLaunchKernelGGL(probe_mfma_lds_kernel<0>, dim3(blocks), dim3(kThreads), 0, s, o, iters); break;
    case 1: hipLaunchKernelGGL(probe_mfma_lds_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, o, iters); break;
    case 2: hipLaunchKernelGGL(probe_mfma_lds_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, o, iters); break;
    case 4: hipLaunchKernelGGL(probe_mfma_lds_kernel<4>, dim3(blocks), dim3(kThreads), 0, s, o, iters); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
