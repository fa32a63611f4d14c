// Small wave-level helpers shared by the GDN kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace spec {
namespace gdn {

template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the wave, the same bits in every lane: within rows of 16 by DPP,
// then across rows and halves by permlane swaps.
__device__ inline float wave_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x * sigmoid(x) with the hardware exponential and reciprocal (about 1 ulp each)
__device__ inline float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

}  // namespace gdn
}  // namespace spec
