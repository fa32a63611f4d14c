// E2E-TV with the teacher logits formed through an output head on MFMA; the
// logits never reach HBM.
//
// [SpecOPD notes page, "Inputs and code mapping"]: prediction logits are read
// from hidden states and a head that the caller supplies, and E2E-TV consumes
// logits aligned by history. [SpecOPD paper page, Figure 3]: the logits of
// step (b,i) come from its predecessor's row (the anchor row for i = 1).
//
//   y[s, v] = <hidden[step_pred_row[s]], head[v]>   bf16 operands, float32 sums
//
// A workgroup (8 waves, two per SIMD, one workgroup per CU) owns a tile of 256
// vocabulary entries x 256 steps and runs the product over the hidden dimension
// in stages of 64 with v_mfma_f32_32x32x16_bf16: vocabulary on the MFMA rows,
// steps on the columns, so a lane's accumulators hold 64 vocabulary entries of
// two steps and every per-step reduction is in-lane plus one exchange with lane
// l ^ 32. Wave w covers vocabulary half w & 1 and step quarter w >> 1 of the
// tile (128 x 64): each fragment read from LDS feeds two or four MFMAs. Both
// operand stages are double-buffered in LDS and filled by buffer loads to LDS
// one stage ahead, in an XOR-swizzled layout that the fragment reads take
// without bank conflicts.
// The product runs twice, because alpha needs the teacher's normaliser before
// any min(q, p) can be summed:
//   pass 1   per (step, 64-entry vocabulary slice): the maximum and the sum of
//            2^(x log2 e - max) of teacher and draft logits
//   merge    per step, slices in order: log2-domain log-sum-exps
//   pass 2   per (step, slice): alpha = sum 2^min(z', y'), S = sum over
//            {z' < y'} of 2^z', and the {q < p} bits
//   sum      per step, slices in order: alpha and S
// and the scan and gradient stages of the supplied-logit path finish it.
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "common.h"

namespace spec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int HT = 256;     // vocabulary entries, and steps, per workgroup tile
constexpr int HK = 64;      // hidden dimensions per product stage
constexpr int HS = 64;      // vocabulary entries per partial slice
constexpr int HGROUP = 8;   // the walk takes tiles in groups of 8 vocabulary tiles x every step tile
constexpr int HSTAGE = HT * HK;  // elements of one operand stage (32 KB)
constexpr float kL2e = 1.4426950408889634f;
constexpr int kHeadWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters at their maxima

// raw buffer descriptor over `bytes` bytes from `base` (reads past the end return zero)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float no_nan(float z) { return __builtin_isnan(z) ? -INFINITY : z; }

// m, s: a running maximum and sum of 2^(x - m); merges (m2, s2) into it
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f(m - mm) + s2 * __builtin_amdgcn_exp2f(m2 - mm);
  m = mm;
}

// One operand stage: 256 rows x 64 hidden dims. The 16-byte chunk c of row r
// sits in slot 8 r + (c ^ swz(r)): 16 consecutive rows read at one chunk fall in
// 16 distinct bank groups (and any aligned 8 of them in 8).
__device__ __forceinline__ int head_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct HeadLds {
  __bf16 a[2][HSTAGE];  // head rows (vocabulary entries)
  __bf16 b[2][HSTAGE];  // hidden rows (the steps' predecessor rows)
};

struct HeadArgs {
  const __bf16 *hidden;
  const int32_t *pred_row;
  const __bf16 *head;
  const void *draft;
  int64_t R, V, n_rows;
  int32_t d, n_vt, n_rt, n_tiles, per_xcd, n_slices;
  float4 *lse_part;  // pass 1 out: [R][n_slices] (max z', sum z', max y', sum y'), log2 units
  const float *lse_q2, *lse_p2;
  float2 *tv_part;   // pass 2 out: [R][n_slices] (alpha, S)
  uint32_t *bits;    // pass 2 out: [R][bits_words], bit u of a row set iff q_u < p_u
  int64_t bits_words;
};

// four consecutive draft logits, held raw until the epilogue widens them
template <typename T> struct Draft4;
template <> struct Draft4<__bf16> {
  uint2 u;
  __device__ __forceinline__ void load(const __bf16 *p) { u = *reinterpret_cast<const uint2 *>(p); }
  __device__ __forceinline__ void clear() { u = make_uint2(0xFF80FF80u, 0xFF80FF80u); }  // -inf
  __device__ __forceinline__ float operator[](int i) const {
    const uint32_t x = i < 2 ? u.x : u.y;
    return __uint_as_float(i & 1 ? x & 0xFFFF0000u : x << 16);
  }
};
template <> struct Draft4<float> {
  float4 f;
  __device__ __forceinline__ void load(const float *p) { f = *reinterpret_cast<const float4 *>(p); }
  __device__ __forceinline__ void clear() { f = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY); }
  __device__ __forceinline__ float operator[](int i) const {
    return i == 0 ? f.x : i == 1 ? f.y : i == 2 ? f.z : f.w;
  }
};

template <typename T, bool PASS2>
__device__ __forceinline__ void head_tile(const HeadArgs &a) {
  __shared__ __attribute__((aligned(16))) HeadLds sm;
  // Workgroups 8 apart run on one XCD; each XCD walks a contiguous run of the
  // tile order, in which groups of 8 vocabulary tiles take every step tile
  // (vocabulary fastest), so the 32 workgroups resident on an XCD share 8 head
  // tiles and 4 hidden tiles in its L2.
  const int t = (blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
  if (t >= a.n_tiles) return;
  const int per_group = HGROUP * a.n_rt;
  const int first_v = t / per_group * HGROUP;
  const int gsize = min(a.n_vt - first_v, HGROUP);
  const int vt = first_v + (t % per_group) % gsize;
  const int rt = (t % per_group) / gsize;
  const int64_t v0 = (int64_t)vt * HT, r0 = (int64_t)rt * HT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS copy bases go to M0
  const int n = lane & 31, half = lane >> 5;
  const int wv = w & 1, wr = w >> 1;  // vocabulary half, step quarter

  // Copies: wave w issues copies q = w + 8 i (i < 4) of each operand stage;
  // copy q fills slots 64 q .. 64 q + 63, i.e. rows 8 q + lane / 8, and lane
  // takes the chunk its slot holds. Rows past the vocabulary or the steps
  // repeat the last one (never stored). The copies are buffer loads to LDS (the
  // head tile's rows and the hidden rows are one buffer each, the stage a
  // scalar offset): outstanding, they leave the LDS counter to the fragment
  // reads, so a wait for one k-step's fragments does not wait for the next's.
  const int cpy_c = (lane & 7) ^ (lane >> 3) ^ (w & 1);
  const int64_t v_rows = min<int64_t>(a.V - v0, HT);
  // the head tile's descriptor, in scalar registers (the compiler cannot see
  // that v0 is the same in every lane)
  const uint64_t abase = (uint64_t)(a.head + v0 * a.d);
  const uint32_t alo = __builtin_amdgcn_readfirstlane((uint32_t)abase);
  const uint32_t ahi = __builtin_amdgcn_readfirstlane((uint32_t)(abase >> 32));
  const uint32_t abytes = __builtin_amdgcn_readfirstlane((uint32_t)(v_rows * a.d * 2));
  const __amdgpu_buffer_rsrc_t rsa =
      head_rsrc(reinterpret_cast<const void *>(((uint64_t)ahi << 32) | alo), abytes);
  const __amdgpu_buffer_rsrc_t rsb = head_rsrc(a.hidden, (uint32_t)(a.n_rows * a.d * 2));
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 64 * i + 8 * w + (lane >> 3);
    const int64_t vr = min<int64_t>(row, v_rows - 1);
    const int64_t r = min<int64_t>(r0 + row, a.R - 1);
    oa[i] = (uint32_t)((vr * a.d + 8 * cpy_c) * 2);
    ob[i] = (uint32_t)(((int64_t)a.pred_row[r] * a.d + 8 * cpy_c) * 2);
  }
  auto copy_stage = [&](int kt, int buf) {
    const uint32_t so = (uint32_t)kt * HK * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = w + 8 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, &sm.a[buf][q * 512], 16, oa[i], so, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, &sm.b[buf][q * 512], 16, ob[i], so, 0, 0);
    }
  };

  f32x16 acc[4][2];  // [vocabulary block i][step block j]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment rows 128 wv + 32 i + n (head) and 64 wr + 32 j + n (hidden): the
  // swizzle depends on n only
  const int swz = head_swz(n);
  const int nk = a.d / HK;
  copy_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(kHeadWaitVm0);
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int cb = kt & 1;
    if (kt + 1 < nk) copy_stage(kt + 1, cb ^ 1);
    __builtin_amdgcn_sched_barrier(0);  // the copies go out before this stage's products
    // fragments of k-step ks + 1 are read before k-step ks's 8 MFMAs are
    // issued (scheduling barriers keep the compiler from sinking the reads to
    // their use), so their LDS latency overlaps the products
    bf16x8 fa[2][4], fb[2][2];
    auto read_frags = [&](int ks, bf16x8 (&xa)[4], bf16x8 (&xb)[2]) {
      const int slot = (2 * ks + half) ^ swz;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xa[i] = *reinterpret_cast<const bf16x8 *>(&sm.a[cb][((128 * wv + 32 * i + n) * 8 + slot) * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        xb[j] = *reinterpret_cast<const bf16x8 *>(&sm.b[cb][((64 * wr + 32 * j + n) * 8 + slot) * 8]);
    };
    read_frags(0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < HK / 16; ++ks) {
      if (ks + 1 < HK / 16) read_frags(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // the reads go out before this k-step's products
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(kHeadWaitVm0);  // this wave's copies of the next stage landed
    __syncthreads();
  }

  // Epilogue. Accumulator e of block (i, j) is the teacher logit of vocabulary
  // entry v0 + 128 wv + 32 i + 8 (e / 4) + 4 half + e % 4 for step
  // r0 + 64 wr + 32 j + n; slice s of the wave's 128 entries is blocks 2s, 2s+1.
  const T *draft = static_cast<const T *>(a.draft);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t row = r0 + 64 * wr + 32 * j + n;
    const int64_t rc = row < a.R ? row : a.R - 1;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int slice = (int)(v0 / HS) + 2 * wv + sl;
      const bool slice_live = (int64_t)slice * HS < a.V;
      const bool store = half == 0 && row < a.R && slice_live;
      Draft4<T> dz[2][4];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t v = v0 + 128 * wv + 32 * (2 * sl + ii) + 8 * g + 4 * half;
          if (v < a.V)
            dz[ii][g].load(draft + rc * a.V + v);
          else
            dz[ii][g].clear();
        }
      if (!PASS2) {
        float my = -INFINITY, mz = -INFINITY;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const bool live = v0 + 128 * wv + 32 * (2 * sl + ii) + 8 * (e / 4) + 4 * half < a.V;
            const float zz = no_nan(dz[ii][e / 4][e % 4]) * kL2e;
            my = fmaxf(my, live ? acc[2 * sl + ii][j][e] * kL2e : -INFINITY);
            mz = fmaxf(mz, zz);
          }
        my = fmaxf(my, __shfl_xor(my, 32));
        mz = fmaxf(mz, __shfl_xor(mz, 32));
        const float my0 = my == -INFINITY ? 0.f : my, mz0 = mz == -INFINITY ? 0.f : mz;
        float sy = 0.f, sz = 0.f;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const bool live = v0 + 128 * wv + 32 * (2 * sl + ii) + 8 * (e / 4) + 4 * half < a.V;
            if (live) sy += __builtin_amdgcn_exp2f(fmaf(acc[2 * sl + ii][j][e], kL2e, -my0));
            sz += __builtin_amdgcn_exp2f(fmaf(no_nan(dz[ii][e / 4][e % 4]), kL2e, -mz0));
          }
        sy += __shfl_xor(sy, 32);
        sz += __shfl_xor(sz, 32);
        if (store) a.lse_part[row * a.n_slices + slice] = make_float4(mz, sz, my, sy);
      } else {
        const float lz = a.lse_q2[rc], ly = a.lse_p2[rc];
        float al = 0.f, ss = 0.f;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int64_t vb = v0 + 128 * wv + 32 * (2 * sl + ii);
          uint32_t word = 0u;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const bool live = vb + 8 * (e / 4) + 4 * half + e % 4 < a.V;
            const float zq = fmaf(no_nan(dz[ii][e / 4][e % 4]), kL2e, -lz);  // log2 q
            const float yp = fmaf(acc[2 * sl + ii][j][e], kL2e, -ly);         // log2 p
            if (live) {
              al += __builtin_amdgcn_exp2f(fminf(zq, yp));
              if (zq < yp) {
                ss += __builtin_amdgcn_exp2f(zq);
                word |= 1u << (8 * (e / 4) + 4 * half + e % 4);
              }
            }
          }
          word |= __shfl_xor(word, 32);
          if (store && vb < a.V) a.bits[row * a.bits_words + vb / 32] = word;
        }
        al += __shfl_xor(al, 32);
        ss += __shfl_xor(ss, 32);
        if (store) a.tv_part[row * a.n_slices + slice] = make_float2(al, ss);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void e2etv_head_lse_kernel(HeadArgs a) {
  head_tile<T, false>(a);
}
template <typename T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void e2etv_head_tv_kernel(HeadArgs a) {
  head_tile<T, true>(a);
}

// One wave per step: merges the step's slice partials in slice order (lane j
// takes slices j, j + 64, ...; then a butterfly, which is order-independent
// because each merge is commutative) into log2-domain log-sum-exps. Workgroup
// 0 also clears the scan's ticket.
__global__ __launch_bounds__(256) void e2etv_head_merge_kernel(const float4 *__restrict__ part,
                                                               int64_t R, int32_t n_slices,
                                                               float *__restrict__ lse_q2,
                                                               float *__restrict__ lse_p2,
                                                               unsigned *__restrict__ ticket) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *ticket = 0u;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  float mz = -INFINITY, sz = 0.f, my = -INFINITY, sy = 0.f;
  for (int j = lane; j < n_slices; j += 64) {
    const float4 p = part[row * n_slices + j];
    lse_merge(mz, sz, p.x, p.y);
    lse_merge(my, sy, p.z, p.w);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float omz = __shfl_xor(mz, off), osz = __shfl_xor(sz, off);
    const float omy = __shfl_xor(my, off), osy = __shfl_xor(sy, off);
    lse_merge(mz, sz, omz, osz);
    lse_merge(my, sy, omy, osy);
  }
  if (lane == 0) {
    lse_q2[row] = mz + __log2f(sz);
    lse_p2[row] = my + __log2f(sy);
  }
}

// One wave per step: sums the step's (alpha, S) slice partials (lane j takes
// slices j, j + 64, ... in order; then a butterfly, whose sums are the same on
// every lane) into one pair, so the scan reads one partial per step.
__global__ __launch_bounds__(256) void e2etv_head_sum_kernel(const float2 *__restrict__ part,
                                                             int64_t R, int32_t n_slices,
                                                             float2 *__restrict__ total) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  float al = 0.f, ss = 0.f;
  for (int j = lane; j < n_slices; j += 64) {
    const float2 p = part[row * n_slices + j];
    al += p.x;
    ss += p.y;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    al += __shfl_xor(al, off);
    ss += __shfl_xor(ss, off);
  }
  if (lane == 0) total[row] = make_float2(al, ss);
}

struct HeadOffsets {
  size_t step, part, status, bsum, bits, total;
  int64_t n_slices, bits_row;
};

// Workspace: four float arrays [R]; the slice partials [R][n_slices] (float4
// in pass 1; in pass 2 float2, followed by the per-step sums [R]); the status words; the per-branch
// sums [R] (float64); the bitmask [R][bits_row].
HeadOffsets head_offsets(int64_t R, int64_t V) {
  HeadOffsets o;
  o.n_slices = (V + HS - 1) / HS;
  o.bits_row = (int64_t)align_up((size_t)(V + 7) / 8, 16);
  o.step = align_up((size_t)R * sizeof(float), 256);
  o.part = 4 * o.step;
  o.status = o.part + align_up((size_t)R * (o.n_slices + 1) * sizeof(float4), 256);
  o.bsum = o.status + 256;
  o.bits = o.bsum + align_up((size_t)R * sizeof(double), 256);
  o.total = o.bits + align_up((size_t)R * o.bits_row, 256);
  return o;
}

template <typename T>
hipError_t run_head(const spec_tree_layout &L, int64_t V, int32_t d, const void *draft,
                    const void *hidden, const void *head, float w, float *alpha, float *loss,
                    float *grad, void *work, hipStream_t s) {
  const int64_t R = L.n_steps;
  const HeadOffsets o = head_offsets(R, V);
  char *p = static_cast<char *>(work);
  E2etvWork ws{};
  ws.lse_q2 = reinterpret_cast<float *>(p);
  ws.lse_p2 = reinterpret_cast<float *>(p + o.step);
  ws.S = reinterpret_cast<float *>(p + 2 * o.step);
  ws.coef = reinterpret_cast<float *>(p + 3 * o.step);
  float2 *slices = reinterpret_cast<float2 *>(p + o.part);
  ws.part = slices + R * o.n_slices;  // the per-step sums the scan reads
  ws.status = reinterpret_cast<unsigned *>(p + o.status);
  ws.branch_sum = reinterpret_cast<double *>(p + o.bsum);
  ws.bits = reinterpret_cast<uint8_t *>(p + o.bits);
  ws.bits_row = o.bits_row;

  HeadArgs a{};
  a.hidden = static_cast<const __bf16 *>(hidden);
  a.pred_row = L.step_pred_row;
  a.head = static_cast<const __bf16 *>(head);
  a.draft = draft;
  a.R = R;
  a.n_rows = L.n_rows;
  a.V = V;
  a.d = d;
  a.n_vt = (int32_t)((V + HT - 1) / HT);
  a.n_rt = (int32_t)((R + HT - 1) / HT);
  const int64_t tiles = (int64_t)a.n_vt * a.n_rt;
  if (tiles > INT32_MAX / 2) return hipErrorInvalidValue;
  a.n_tiles = (int32_t)tiles;
  a.per_xcd = (int32_t)((tiles + 7) / 8);
  a.n_slices = (int32_t)o.n_slices;
  a.lse_part = reinterpret_cast<float4 *>(p + o.part);
  a.lse_q2 = ws.lse_q2;
  a.lse_p2 = ws.lse_p2;
  a.tv_part = slices;
  a.bits = reinterpret_cast<uint32_t *>(ws.bits);
  a.bits_words = o.bits_row / 4;
  const dim3 grid((unsigned)(8 * (int64_t)a.per_xcd));

  hipLaunchKernelGGL((e2etv_head_lse_kernel<T>), grid, dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_head_lse");
  hipLaunchKernelGGL(e2etv_head_merge_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s,
                     a.lse_part, R, a.n_slices, ws.lse_q2, ws.lse_p2, ws.status + 1);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_head_merge");
  hipLaunchKernelGGL((e2etv_head_tv_kernel<T>), grid, dim3(512), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_head_tv");
  hipLaunchKernelGGL(e2etv_head_sum_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s,
                     slices, R, a.n_slices, ws.part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_mark(s, "e2etv_head_sum");
  return launch_e2etv_tail(L, V, std::is_same<T, __bf16>::value ? SPEC_BF16 : SPEC_F32, draft, w, 1,
                           alpha, loss, grad, ws, s);
}

}  // namespace

size_t e2etv_head_work_bytes(int64_t R, int64_t V) { return head_offsets(R, V).total; }

hipError_t launch_e2etv_head(const spec_tree_layout &L, int64_t V, int32_t d, spec_dtype dtype,
                             const void *draft, const void *hidden, const void *head, float w,
                             float *alpha, float *loss, float *grad, void *work, hipStream_t s) {
  return dtype == SPEC_BF16
             ? run_head<__bf16>(L, V, d, draft, hidden, head, w, alpha, loss, grad, work, s)
             : run_head<float>(L, V, d, draft, hidden, head, w, alpha, loss, grad, work, s);
}

}  // namespace spec
