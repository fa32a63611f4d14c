// Tree-masked GQA attention over a packed proposal tree, plus readout.
//
// [SpecOPD paper page, Figure 3]: packed queries share the trunk K/V and every
// row attends to itself and its ancestors only.
// [SpecOPD notes page, "Equations"]: a branch row sees the reference prefix
// through its anchor and its own branch predecessors; the anchor row predicts
// y_{b,1} and the row of y_{b,i-1} predicts y_{b,i} (never the sample's own row).
//
// bf16 path (CDNA4 MFMA). A workgroup owns one query block of <= 32 packed rows
// (an AttnItem) for one KV head g and NW of the query heads that share it; wave
// w handles query head h = g*G + w for the 32 rows, so the K/V tiles staged in
// LDS serve NW heads. The key loop runs over the block's trunk range, then its
// branch range, in tiles of 64 keys:
//   S^T[key][query] = K Q^T     v_mfma_f32_32x32x16_bf16, 2 output tiles x D/16 steps
//   online softmax  per query column, in-lane over 32 keys + one cross-half max;
//                   the reference maximum moves only when a score exceeds it by
//                   more than 2^8, so the output is rarely rescaled
//   O^T[d][query]  += V^T P^T   D/32 output tiles x 4 steps
// Keys on the rows, queries on the columns keeps each query's scores, max and
// sum inside one lane (plus its partner lane l^32), and lets the probabilities
// feed the second MFMA straight from registers: the V^T tile in LDS stores its
// 16-key groups as key quads [0, 2, 1, 3] so that a lane's 8 B-operand slots
// line up with the keys its accumulator holds. Tiles that every query of the
// block sees in full skip the mask; the rest compare the key against the
// query's two visible intervals. Rows of Q are rotated in registers on load.
// Head dims 32 and 64 stage K and V through registers (tree_attn_bf16_kernel);
// head dim 128 copies 64-key tiles that a pre-pass laid out in the fragments'
// LDS order straight into LDS (tree_attn_tiled_kernel, below). The tiled kernel
// forms the exponentials before any maximum, against the current reference, and
// forms the tile maximum only when a partial sum shows a probability above
// 2^8 (or the reference is still unset): the decisions, and so the outputs, are
// those of the maximum-first order, with the maxima left out of the usual tile.
//
// fp32 path: one wavefront per (row, head) walks the visible keys in order with
// an exact float32 online softmax (no MFMA); it serves float32 inputs.
#include "common.h"

namespace spec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KT = 64;  // keys per tile
constexpr float kLazyMax = 8.f;  // log2 headroom of the softmax reference

template <int D>
struct AttnSmem {
  __bf16 k[KT][D + 8];   // K tile, row-major, padded against bank conflicts
  __bf16 vt[D][KT + 8];  // V tile transposed, key quads permuted
};

// Global -> register -> LDS staging of one 64-key tile of KV head g: the loads
// of the next tile are issued before the current tile is computed (registers
// hold them), and the LDS tiles are double-buffered, so one barrier per tile
// suffices. Keys past `ke` read as zero.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int D, int NT>
struct TileRegs {
  static constexpr int CH = D / 8;                       // 16-byte chunks per row
  static constexpr int KPT = (KT * CH + NT - 1) / NT;    // K chunks per thread
  static constexpr int VPT = (16 * CH + NT - 1) / NT;    // V (key quad, chunk) tasks per thread
  uint4 k[KPT];
  uint4 v[VPT][4];

  // Buffer loads whose descriptor ends at key `ke`: keys past it read as zero
  // without any per-load condition.
  __device__ inline void load(const __bf16 *__restrict__ kws, const __bf16 *__restrict__ vv, int g,
                              int hkv, int64_t n_rows, int k0, int ke, int tid) {
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(kws + (int64_t)g * n_rows * D, (uint32_t)ke * D * 2);
    const uint32_t vrow = (uint32_t)hkv * D * 2;  // bytes between consecutive keys of V
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(vv + (int64_t)g * D, ke > 0 ? (uint32_t)(ke - 1) * vrow + D * 2 : 0u);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      const uint32_t off = ((uint32_t)(k0 + c / CH) * D + (c % CH) * 8) * 2;
      k[i] = (KPT * NT == KT * CH || c < KT * CH) ? load16(rk, off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      const int kq = c % 16, col = c / 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t off = (uint32_t)(k0 + 4 * kq + e) * vrow + col * 16;
        v[i][e] = (VPT * NT == 16 * CH || c < 16 * CH) ? load16(rv, off) : make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ inline void store(AttnSmem<D> &sm, int tid) const {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (c < KT * CH) *reinterpret_cast<uint4 *>(&sm.k[c / CH][(c % CH) * 8]) = k[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      if (c >= 16 * CH) continue;
      const int kq = c % 16, col = c / 16;
      // quad kq of its 16-key group goes to slot {0, 8, 4, 12}[kq % 4]
      const int pos = 16 * (kq >> 2) + ((kq & 1) << 3) + ((kq & 2) << 1);
      const uint32_t w[4][4] = {{v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w},
                                {v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w},
                                {v[i][2].x, v[i][2].y, v[i][2].z, v[i][2].w},
                                {v[i][3].x, v[i][3].y, v[i][3].z, v[i][3].w}};
#pragma unroll
      for (int x = 0; x < 4; ++x) {  // dims 2x (low halves) and 2x+1 (high halves)
        uint2 lo, hi;
        lo.x = (w[0][x] & 0xffffu) | (w[1][x] << 16);
        lo.y = (w[2][x] & 0xffffu) | (w[3][x] << 16);
        hi.x = (w[0][x] >> 16) | (w[1][x] & 0xffff0000u);
        hi.y = (w[2][x] >> 16) | (w[3][x] & 0xffff0000u);
        *reinterpret_cast<uint2 *>(&sm.vt[col * 8 + 2 * x][pos]) = lo;
        *reinterpret_cast<uint2 *>(&sm.vt[col * 8 + 2 * x + 1][pos]) = hi;
      }
    }
  }
};

// max / sum over the lane pair (l, l ^ 32), identical in both lanes
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two waves per SIMD where the LDS allows it (four or more waves per workgroup);
// with one or two waves per workgroup the double-buffered tiles already cap a CU
// at one wave per SIMD, so only that is asked for.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW >= 4 ? 2 : 1, 2))) void tree_attn_bf16_kernel(
    const AttnItem *__restrict__ items, int hkv, int group, int hsub,
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kws, const __bf16 *__restrict__ v,
    __bf16 *__restrict__ out, const float2 *__restrict__ tab, const int32_t *__restrict__ row_pos,
    const int32_t *__restrict__ row_trunk_hi, const int32_t *__restrict__ row_branch_lo,
    int64_t n_rows, int hq, float sl2) {
  constexpr int NT = NW * 64;
  constexpr int KS = D / 16;  // contraction steps of Q K^T
  constexpr int DT = D / 32;  // output tiles of P V
  __shared__ AttnSmem<D> sm[2];

  // block -> (item, kv head, head slice). Consecutive blocks cycle over KV heads,
  // so with the round-robin dispatch over XCDs each XCD keeps to few heads.
  const int bid = blockIdx.x;
  const int g = bid % hkv;
  const int rest = bid / hkv;
  const int hs = rest % hsub;
  const AttnItem it = items[rest / hsub];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = lane & 31, half = lane >> 5;
  const int hl = hs * NW + w;
  const bool active = hl < group;  // wave-uniform
  const int h = g * group + (active ? hl : 0);
  const int qrow = min(it.q0 + n, it.q1 - 1);  // padding columns repeat the last row

  // tiles: trunk keys [tk0, tk1) then branch keys [bk0, bk1), 64 keys each
  const int n_trunk = (it.tk1 - it.tk0 + KT - 1) / KT;
  const int n_tiles = n_trunk + (it.bk1 - it.bk0 + KT - 1) / KT;
  auto tile_k0 = [&](int t) { return t < n_trunk ? it.tk0 + KT * t : it.bk0 + KT * (t - n_trunk); };
  auto tile_ke = [&](int t) { return t < n_trunk ? it.tk1 : it.bk1; };

  TileRegs<D, NT> regs;
  if (n_tiles > 0) regs.load(kws, v, g, hkv, n_rows, tile_k0(0), tile_ke(0), tid);

  // Q for this lane's query column, rotated and pre-scaled by scale*log2(e):
  // k-step s holds dims 16s + 8*half + [0, 8)
  bf16x8 qf[KS];
  {
    const __bf16 *qp = q + ((int64_t)qrow * hq + h) * D;
    const float2 *tp = tab + (int64_t)row_pos[qrow] * (D / 2);
#pragma unroll
    for (int s = 0; s < KS / 2; ++s) {
      const int d0 = 16 * s + 8 * half;  // first half; partner dims are d0 + D/2
      const bf16x8 x1 = *reinterpret_cast<const bf16x8 *>(qp + d0);
      const bf16x8 x2 = *reinterpret_cast<const bf16x8 *>(qp + d0 + D / 2);
      bf16x8 y1, y2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 cs = tp[d0 + j];
        const float a = (float)x1[j], b = (float)x2[j];
        y1[j] = (__bf16)((a * cs.x - b * cs.y) * sl2);
        y2[j] = (__bf16)((b * cs.x + a * cs.y) * sl2);
      }
      qf[s] = y1;
      qf[s + KS / 2] = y2;
    }
  }
  // this query's visible keys: [tree start, thi] U [blo, qrow]
  const int thi = row_trunk_hi[qrow];
  const int blo = row_branch_lo[qrow];
  const int bhi = qrow;

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  // m: the softmax reference of this lane's query (log2 units); the score
  // MFMAs start from -m_use, so they produce s - m_use directly
  float m = -INFINITY, l = 0.f;
  f32x16 negm;
#pragma unroll
  for (int i = 0; i < 16; ++i) negm[i] = 0.f;

  // O^T += V^T P^T for one tile's probabilities p and V^T tile vt
  auto pv = [&](const AttnSmem<D> &vt, const bf16x8 (&p)[4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&vt.vt[32 * dt + n][16 * kk + 8 * half]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[kk], o[dt], 0, 0, 0);
      }
  };

  // Software pipeline: the P V product of a tile runs one tile late, beside the
  // next tile's exponentials (the two take about the same time), so each tile is
  //   S(t), softmax(t) with O += V(t-1) P(t-1) | barrier | stage tile t+1 | barrier.
  // Before the first tile the "previous" probabilities are zero and the other
  // V^T buffer is cleared, so that product adds nothing.
  bf16x8 pp[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) pp[kk][e] = (__bf16)0.f;
  if (n_tiles > 0) regs.store(sm[0], tid);
  for (int i = tid; i < (int)(sizeof(sm[1].vt) / 16); i += NT)
    reinterpret_cast<uint4 *>(&sm[1].vt[0][0])[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  if (n_tiles > 1) regs.load(kws, v, g, hkv, n_rows, tile_k0(1), tile_ke(1), tid);

  for (int t = 0; t < n_tiles; ++t) {
    AttnSmem<D> &cur = sm[t & 1];
    AttnSmem<D> &prv = sm[(t + 1) & 1];  // tile t - 1, then the staging buffer of tile t + 1
    const int k0 = tile_k0(t);
    const bool branch = t >= n_trunk;
    if (active) {
      f32x16 s0 = negm, s1 = negm;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(&cur.k[n][16 * s + 8 * half]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(&cur.k[32 + n][16 * s + 8 * half]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], s1, 0, 0, 0);
      }
      // accumulator i of tile t holds key k0 + 32t + 8(i/4) + 4*half + i%4; a lane sees the
      // keys [vlo, vhi] of this range (its trunk prefix, or its own branch run)
      const bool need_mask = branch || (k0 + KT > it.tfull);
      if (need_mask) {
        const int vlo = branch ? blo : it.tk0, vhi = branch ? bhi : thi;
        const uint32_t span = (uint32_t)(vhi - vlo);
        const int base = k0 + 4 * half - vlo;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o0 = base + 8 * (i >> 2) + (i & 3);
          s0[i] = (uint32_t)o0 <= span ? s0[i] : -INFINITY;
          s1[i] = (uint32_t)(o0 + 32) <= span ? s1[i] : -INFINITY;
        }
      }
      // three-input maxima: 16 instructions for the 32 scores of the lane
      auto max3 = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
      float ma[5], mb[5];
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        ma[k] = max3(s0[3 * k], s0[3 * k + 1], s0[3 * k + 2]);
        mb[k] = max3(s1[3 * k], s1[3 * k + 1], s1[3 * k + 2]);
      }
      const float mc = max3(s0[15], s1[15], ma[0]);
      const float md = max3(ma[1], ma[2], ma[3]), me = max3(ma[4], mb[0], mb[1]), mf = max3(mb[2], mb[3], mb[4]);
      const float m_use = m == -INFINITY ? 0.f : m;
      const float mx = pair_max(fmaxf(max3(mc, md, me), mf)) + m_use;
      // The reference m moves only when a score exceeds it by more than
      // kLazyMax, so O and l are rescaled on few tiles; in between the
      // probabilities are at most 2^kLazyMax.
      if (__any(mx > m + kLazyMax)) {
        pv(prv, pp);  // the previous tile's product, at the old reference
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) pp[kk][e] = (__bf16)0.f;
        const float m_new = mx > m + kLazyMax ? mx : m;
        const float corr = m_new == m ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
        l *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] *= corr;
        m = m_new;
        // re-base this tile's scores and the next tiles' starting value
        const float m_use2 = m == -INFINITY ? 0.f : m;
        const float d = m_use - m_use2;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s0[i] += d;
          s1[i] += d;
          negm[i] = -m_use2;
        }
      }
      float ls0 = 0.f, ls1 = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(s0[i]);
        ls0 += p0;
        pf[i >> 3][i & 7] = (__bf16)p0;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p1 = __builtin_amdgcn_exp2f(s1[i]);
        ls1 += p1;
        pf[2 + (i >> 3)][i & 7] = (__bf16)p1;
      }
      l += ls0 + ls1;
      pv(prv, pp);  // the previous tile's product, beside this tile's exponentials
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pp[kk] = pf[kk];
    }
    __syncthreads();  // every wave is done with tile t - 1
    if (t + 1 < n_tiles) regs.store(prv, tid);
    __syncthreads();
    if (t + 2 < n_tiles) regs.load(kws, v, g, hkv, n_rows, tile_k0(t + 2), tile_ke(t + 2), tid);
  }
  if (active && n_tiles > 0) pv(sm[(n_tiles - 1) & 1], pp);

  const float inv = 1.f / pair_sum(l);
  if (active && it.q0 + n < it.q1) {
    __bf16 *op = out + ((int64_t)(it.q0 + n) * hq + h) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        // accumulator 4*i4 + e holds dim 32t + 8*i4 + 4*half + e
        __bf16 r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = (__bf16)(o[t][4 * i4 + e] * inv);
        uint2 pk;
        __builtin_memcpy(&pk, r4, 8);
        *reinterpret_cast<uint2 *>(op + 32 * t + 8 * i4 + 4 * half) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// Head dim 128 with tiled K and V (kv_tile_kernel): the same block decomposition
// and per-tile math as tree_attn_bf16_kernel, but a 64-key tile is copied
// global -> LDS by direct-to-LDS loads (16 bytes per lane, laid out by the
// pre-pass exactly as the MFMA fragments read them), so staging takes no
// registers and no VALU work. Key tiles are aligned to multiples of 64 in the
// packed order; keys outside a query's visible ranges are masked as before.
// Tile t's work is S(t) = K(t) Q^T, then its exponentials with the previous
// tile's O += V(t-1) P(t-1) issued between them (one MFMA, two exponentials,
// ...), so the matrix core runs while the VALU works. K(t+1) and V(t) are
// copied during tile t into the other K buffer and the V buffer that P V(t-2)
// has finished with: two buffers of each, one wait and one barrier per tile.
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), as an
// immediate the compiler's own wait bookkeeping sees
constexpr int kWaitVm0 = 0x0F70;
constexpr float kLazyLimit = 256.f;  // 2^kLazyMax
static_assert(kLazyMax == 8.f && kLazyLimit == 256.f, "kLazyLimit is 2^kLazyMax");

// NW query heads of one KV head (one wave each) for NB query blocks: NB = 1 takes
// one block of the longest-first list; NB > 1 (one or two query heads per KV head)
// takes NB blocks of a group (consecutive blocks of one tree's trunk or branch
// rows), so that each staged tile serves NW * NB waves. The tiles then cover the
// union of the blocks' key ranges, and a wave's own masks discard the keys its
// rows do not see.
template <int NW, int NB>
__global__ __launch_bounds__(NW * NB * 64) __attribute__((amdgpu_waves_per_eu(NW * NB >= 4 ? 2 : 1, 2))) void tree_attn_tiled_kernel(
    const AttnItem *__restrict__ items, int n_items, int hkv, int group, int hsub,
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kt, const __bf16 *__restrict__ vt,
    __bf16 *__restrict__ out, const float2 *__restrict__ tab, const int32_t *__restrict__ row_pos,
    const int32_t *__restrict__ row_trunk_hi, const int32_t *__restrict__ row_branch_lo,
    int32_t n_key_tiles, int hq, float sl2) {
  constexpr int D = 128, KS = D / 16, DT = D / 32;
  constexpr int NWAVE = NW * NB;
  constexpr int PIECES = KT * D * 2 / 1024;  // 1 KB copies per K (or V^T) tile
  static_assert(PIECES % NWAVE == 0, "each wave issues the same number of copies");
  static_assert(kAttnGroup % NB == 0, "a workgroup takes whole slices of a group");
  // K tiles: slot r*16 + (c ^ (r & 15)) holds dims 8c..8c+7 of key r; V^T tiles:
  // slot d*8 + (c ^ vt_swizzle(d)) holds positions 8c..8c+7 of dim d. Four arrays,
  // so the compiler can see that no fragment read touches a buffer being filled.
  __shared__ __attribute__((aligned(16))) __bf16 kb0[KT * D], kb1[KT * D], vb0[D * KT], vb1[D * KT];

  const int bid = blockIdx.x;
  const int g = bid % hkv;
  const int rest = bid / hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS copy bases go to M0
  const int n = lane & 31, half = lane >> 5;
  const AttnItem *blocks;  // this workgroup's NB blocks
  int hs = 0;
  if constexpr (NB == 1) {
    hs = rest % hsub;
    blocks = items + rest / hsub;
  } else {
    constexpr int PER = kAttnGroup / NB;  // workgroups per group
    blocks = items + n_items + (int64_t)(rest / PER) * kAttnGroup + (rest % PER) * NB;
  }
  const AttnItem it = blocks[w / NW];
  const bool rows = it.q1 > it.q0;  // false for a group's padding
  const int hl = hs * NW + w % NW;
  const bool active = hl < group && rows;  // wave-uniform
  const int h = g * group + (active ? hl : 0);
  const int qrow = rows ? min(it.q0 + n, it.q1 - 1) : 0;

  // 64-aligned key tiles over the union of the blocks' ranges: trunk tiles cover
  // [tk0, tk1), then branch tiles [bk0, bk1)
  int tt0 = 0, tt1 = 0, bt0 = 0, bt1 = 0;
  {
    bool any_t = false, any_b = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const AttnItem x = blocks[b];
      if (x.q1 <= x.q0) continue;
      if (x.tk1 > x.tk0) {
        const int a0 = x.tk0 / KT, a1 = (x.tk1 - 1) / KT + 1;
        tt0 = any_t ? min(tt0, a0) : a0;
        tt1 = any_t ? max(tt1, a1) : a1;
        any_t = true;
      }
      if (x.bk1 > x.bk0) {
        const int a0 = x.bk0 / KT, a1 = (x.bk1 - 1) / KT + 1;
        bt0 = any_b ? min(bt0, a0) : a0;
        bt1 = any_b ? max(bt1, a1) : a1;
        any_b = true;
      }
    }
  }
  const int n_trunk = tt1 - tt0;
  const int n_tiles = n_trunk + (bt1 - bt0);
  auto tile_index = [&](int t) { return t < n_trunk ? tt0 + t : bt0 + (t - n_trunk); };

  // copy the K (or V^T) half of tile t into `dst`: wave w issues the 1 KB pieces
  // w, w + NWAVE, ... as buffer loads to LDS (the KV head's tiles are one buffer, the
  // piece's byte offset a scalar): outstanding, they leave the LDS counter to the
  // fragment reads, which can then be issued ahead and waited for one at a time
  const uint32_t head_bytes = (uint32_t)n_key_tiles * KT * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kt + (int64_t)g * n_key_tiles * KT * D, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vt + (int64_t)g * n_key_tiles * KT * D, head_bytes);
  const uint32_t lane_off = (uint32_t)lane * 16;
  auto copy_k = [&](int t, __bf16 *dst) {
    const uint32_t off = (uint32_t)tile_index(t) * (KT * D * 2);
#pragma unroll
    for (int i = 0; i < PIECES / NWAVE; ++i) {
      const int j = w + NWAVE * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst + j * 512, 16, lane_off, off + (uint32_t)j * 1024, 0, 0);
    }
  };
  auto copy_v = [&](int t, __bf16 *dst) {
    const uint32_t off = (uint32_t)tile_index(t) * (KT * D * 2);
#pragma unroll
    for (int i = 0; i < PIECES / NWAVE; ++i) {
      const int j = w + NWAVE * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst + j * 512, 16, lane_off, off + (uint32_t)j * 1024, 0, 0);
    }
  };

  // per-row inputs first: the RoPE table row depends on row_pos
  const int pos = row_pos[qrow];
  int thi = row_trunk_hi[qrow];
  int blo = row_branch_lo[qrow];
  if (n_tiles > 0) copy_k(0, kb0);

  bf16x8 qf[KS];
  {
    const __bf16 *qp = q + ((int64_t)qrow * hq + h) * D;
    const float2 *tp = tab + (int64_t)pos * (D / 2);
#pragma unroll
    for (int s = 0; s < KS / 2; ++s) {
      const int d0 = 16 * s + 8 * half;
      const bf16x8 x1 = *reinterpret_cast<const bf16x8 *>(qp + d0);
      const bf16x8 x2 = *reinterpret_cast<const bf16x8 *>(qp + d0 + D / 2);
      bf16x8 y1, y2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 cs = tp[d0 + j];
        const float a = (float)x1[j], b = (float)x2[j];
        y1[j] = (__bf16)((a * cs.x - b * cs.y) * sl2);
        y2[j] = (__bf16)((b * cs.x + a * cs.y) * sl2);
      }
      qf[s] = y1;
      qf[s + KS / 2] = y2;
    }
  }
  // kept in registers and computed here, beside the first tile copy: left to
  // itself the compiler sinks the Q loads and rotation behind the first
  // barrier, and a reload of thi/blo inside the tile loop would wait for the
  // tile copies in flight
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 r = __builtin_bit_cast(u32x4, qf[s]);
    asm volatile("" : "+v"(r));
    qf[s] = __builtin_bit_cast(bf16x8, r);
  }
  asm volatile("" : "+v"(thi), "+v"(blo));
  const int bhi = qrow;

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m = -INFINITY, l = 0.f;
  f32x16 negm;
#pragma unroll
  for (int i = 0; i < 16; ++i) negm[i] = 0.f;
  bf16x8 pp[4];  // the previous tile's probabilities

  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  auto read_v = [&](const __bf16 *vs, int x) {
    const int kk = x / DT, dt = x % DT;
    const int row = 32 * dt + n, c = 2 * kk + half;
    return *reinterpret_cast<const bf16x8 *>(&vs[(row * 8 + (c ^ vt_swizzle(row))) * 8]);
  };
  // O^T += V^T P^T over one tile, V^T fragments read one MFMA ahead
  auto pv = [&](const __bf16 *vs, const bf16x8 (&p)[4]) {
    bf16x8 va[2];
    va[0] = read_v(vs, 0);
#pragma unroll
    for (int x = 0; x < 4 * DT; ++x) {
      if (x + 1 < 4 * DT) va[(x + 1) & 1] = read_v(vs, x + 1);
      __builtin_amdgcn_sched_barrier(0);
      o[x % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[x & 1], p[x / DT], o[x % DT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // probability of score i (0..31: s0 then s1) into pf, added to its half's sum;
  // the sums run over i in order
  auto prob = [&](const f32x16 &s0, const f32x16 &s1, int i, bf16x8 (&pf)[4], float &ls0, float &ls1) {
    const float p = __builtin_amdgcn_exp2f(i < 16 ? s0[i & 15] : s1[i & 15]);
    if (i < 16)
      ls0 += p;
    else
      ls1 += p;
    pf[i >> 3][i & 7] = (__bf16)p;
  };
  auto exps = [&](const f32x16 &s0, const f32x16 &s1, bf16x8 (&pf)[4], float &ls0, float &ls1) {
    ls0 = 0.f;
    ls1 = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) prob(s0, s1, i, pf, ls0, ls1);
  };
  // the same exponentials with the previous tile's product between them: one
  // MFMA (its V^T fragment read three MFMAs ahead), then two exponentials
  auto exps_pv = [&](const __bf16 *vs, const f32x16 &s0, const f32x16 &s1, bf16x8 (&pf)[4], float &ls0,
                     float &ls1) {
    ls0 = 0.f;
    ls1 = 0.f;
    constexpr int AH = 3;
    bf16x8 va[AH + 1];
#pragma unroll
    for (int x = 0; x < AH; ++x) va[x] = read_v(vs, x);
#pragma unroll
    for (int x = 0; x < 4 * DT; ++x) {
      if (x + AH < 4 * DT) va[(x + AH) % (AH + 1)] = read_v(vs, x + AH);
      __builtin_amdgcn_sched_barrier(0);
      o[x % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[x % (AH + 1)], pp[x / DT], o[x % DT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      prob(s0, s1, 2 * x, pf, ls0, ls1);
      prob(s0, s1, 2 * x + 1, pf, ls0, ls1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto body = [&](int t, const __bf16 *kcur, __bf16 *knext, const __bf16 *vprev, __bf16 *vnext, bool first) {
    if (t + 1 < n_tiles) copy_k(t + 1, knext);
    copy_v(t, vnext);
    __builtin_amdgcn_sched_barrier(0);  // the copies go out before this tile's work
    const int k0 = tile_index(t) * KT;
    const bool branch = t >= n_trunk;
    if (active) {
      f32x16 s0 = negm, s1 = negm;
      // K fragments of step s + 1 are read before step s's MFMAs are issued
      bf16x8 ka[2][2];
      auto read_k = [&](int s, bf16x8 (&x)[2]) {
        const int c = 2 * s + half;
        x[0] = *reinterpret_cast<const bf16x8 *>(&kcur[(n * 16 + (c ^ (n & 15))) * 8]);
        x[1] = *reinterpret_cast<const bf16x8 *>(&kcur[((32 + n) * 16 + (c ^ (n & 15))) * 8]);
      };
      read_k(0, ka[0]);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) read_k(s + 1, ka[(s + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s & 1][0], qf[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s & 1][1], qf[s], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool need_mask = branch || k0 < it.tk0 || (k0 + KT > it.tfull);
      if (need_mask) {
        const int vlo = branch ? blo : it.tk0, vhi = branch ? bhi : thi;
        const uint32_t span = (uint32_t)(vhi - vlo);
        const int base = k0 + 4 * half - vlo;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o0 = base + 8 * (i >> 2) + (i & 3);
          s0[i] = (uint32_t)o0 <= span ? s0[i] : -INFINITY;
          s1[i] = (uint32_t)(o0 + 32) <= span ? s1[i] : -INFINITY;
        }
      }
      // Exponentials against the current reference m first (the previous tile's
      // P V between them, so it is accumulated at the old reference). The
      // reference moves only when a score exceeds it by more than kLazyMax, i.e.
      // when some probability exceeds 2^kLazyMax, and then one of the lane's two
      // partial sums does too; only then (and while m is unset) is the tile's
      // maximum formed, O and l rescaled and the exponentials redone.
      bf16x8 pf[4];
      float ls0, ls1;
      if (first)
        exps(s0, s1, pf, ls0, ls1);
      else
        exps_pv(vprev, s0, s1, pf, ls0, ls1);
      if (__any(fmaxf(ls0, ls1) > kLazyLimit || m == -INFINITY)) {
        auto max3 = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
        float ma[5], mb[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) {
          ma[k] = max3(s0[3 * k], s0[3 * k + 1], s0[3 * k + 2]);
          mb[k] = max3(s1[3 * k], s1[3 * k + 1], s1[3 * k + 2]);
        }
        const float mc = max3(s0[15], s1[15], ma[0]);
        const float md = max3(ma[1], ma[2], ma[3]), me = max3(ma[4], mb[0], mb[1]), mf = max3(mb[2], mb[3], mb[4]);
        const float m_use = m == -INFINITY ? 0.f : m;
        const float mx = pair_max(fmaxf(max3(mc, md, me), mf)) + m_use;
        if (__any(mx > m + kLazyMax)) {
          const float m_new = mx > m + kLazyMax ? mx : m;
          const float corr = m_new == m ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
          l *= corr;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= corr;
          m = m_new;
          const float m_use2 = m == -INFINITY ? 0.f : m;
          const float d = m_use - m_use2;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s0[i] += d;
            s1[i] += d;
            negm[i] = -m_use2;
          }
          exps(s0, s1, pf, ls0, ls1);
        }
      }
      l += ls0 + ls1;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pp[kk] = pf[kk];
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's copies of K(t + 1) and V(t) landed
    __syncthreads();
  };
  if (n_tiles > 0) {
    body(0, kb0, kb1, vb1, vb0, true);
    for (int t = 1; t < n_tiles; t += 2) {
      body(t, kb1, kb0, vb0, vb1, false);
      if (t + 1 < n_tiles) body(t + 1, kb0, kb1, vb1, vb0, false);
    }
    if (active) pv((n_tiles - 1) & 1 ? vb1 : vb0, pp);
  }

  const float inv = 1.f / pair_sum(l);
  if (active && it.q0 + n < it.q1) {
    __bf16 *op = out + ((int64_t)(it.q0 + n) * hq + h) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        __bf16 r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = (__bf16)(o[t][4 * i4 + e] * inv);
        uint2 pk;
        __builtin_memcpy(&pk, r4, 8);
        *reinterpret_cast<uint2 *>(op + 32 * t + 8 * i4 + 4 * half) = pk;
      }
  }
}

// Exact float32 path: one wavefront per (row, head); lane holds dims lane and lane + 64.
template <int D>
__global__ __launch_bounds__(64) void tree_attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ kws, const float *__restrict__ v,
    float *__restrict__ out, const float2 *__restrict__ tab, const int32_t *__restrict__ tree_off,
    const int32_t *__restrict__ row_tree, const int32_t *__restrict__ row_pos,
    const int32_t *__restrict__ row_trunk_hi, const int32_t *__restrict__ row_branch_lo,
    int64_t n_rows, int hq, int hkv, float scale) {
  constexpr int H = D / 2;
  constexpr int PER = D > 64 ? 2 : 1;
  const int r = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int g = h / (hq / hkv);
  const float *qp = q + ((int64_t)r * hq + h) * D;
  const float2 *tp = tab + (int64_t)row_pos[r] * H;
  float qr[PER], o[PER];
  bool on[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = lane + 64 * e;
    on[e] = d < D;
    qr[e] = 0.f;
    o[e] = 0.f;
    if (on[e]) {
      const int j = d < H ? d : d - H;
      const float2 cs = tp[j];
      const float x1 = qp[j], x2 = qp[j + H];
      qr[e] = d < H ? x1 * cs.x - x2 * cs.y : x2 * cs.x + x1 * cs.y;
    }
  }
  float m = -INFINITY, l = 0.f;
  const int lo = tree_off[row_tree[r]], thi = row_trunk_hi[r], blo = row_branch_lo[r];
  for (int phase = 0; phase < 2; ++phase) {
    const int c0 = phase == 0 ? lo : blo;
    const int c1 = phase == 0 ? thi : r;
    for (int c = c0; c <= c1; ++c) {
      const float *kp = kws + ((int64_t)g * n_rows + c) * D;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (on[e]) part += qr[e] * kp[lane + 64 * e];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
      const float s = part * scale;
      const float m_new = fmaxf(m, s);
      const float corr = expf(m - m_new);
      const float p = expf(s - m_new);
      l = l * corr + p;
      const float *vp = v + ((int64_t)c * hkv + g) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (on[e]) o[e] = o[e] * corr + p * vp[lane + 64 * e];
      m = m_new;
    }
  }
  float *op = out + ((int64_t)r * hq + h) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (on[e]) op[lane + 64 * e] = o[e] / l;
}

namespace {

template <int D, int NW>
hipError_t launch_bf16(const spec_tree_layout &L, int hq, int hkv, const void *q, const void *kws,
                       const void *v, const float2 *tab, float scale, void *out, hipStream_t s) {
  const int group = hq / hkv;
  const int hsub = (group + NW - 1) / NW;
  const int64_t nblk = (int64_t)L.n_attn_items * hkv * hsub;
  if (nblk == 0) return hipSuccess;
  if (nblk > INT32_MAX) return hipErrorInvalidValue;
  const float sl2 = scale * 1.4426950408889634f;  // scores in log2 units
  hipLaunchKernelGGL((tree_attn_bf16_kernel<D, NW>), dim3((unsigned)nblk), dim3(NW * 64), 0, s,
                     reinterpret_cast<const AttnItem *>(L.attn_items), hkv, group, hsub,
                     static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(kws),
                     static_cast<const __bf16 *>(v), static_cast<__bf16 *>(out), tab, L.row_pos,
                     L.row_trunk_hi, L.row_branch_lo, L.n_rows, hq, sl2);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(const spec_tree_layout &L, int hq, int hkv, const void *q, const void *kws,
                         const void *v, const float2 *tab, float scale, void *out, hipStream_t s) {
  const int group = hq / hkv;
  if (group >= 8) return launch_bf16<D, 8>(L, hq, hkv, q, kws, v, tab, scale, out, s);
  if (group >= 3) return launch_bf16<D, 4>(L, hq, hkv, q, kws, v, tab, scale, out, s);
  if (group == 2) return launch_bf16<D, 2>(L, hq, hkv, q, kws, v, tab, scale, out, s);
  return launch_bf16<D, 1>(L, hq, hkv, q, kws, v, tab, scale, out, s);
}

template <int NW, int NB>
hipError_t launch_tiled(const spec_tree_layout &L, int hq, int hkv, const void *q, const void *kt,
                        const void *vt, const float2 *tab, float scale, void *out, hipStream_t s) {
  const int group = hq / hkv;
  const int hsub = (group + NW - 1) / NW;
  if (NB > 1 && hsub != 1) return hipErrorInvalidValue;
  const int64_t units = NB == 1 ? (int64_t)L.n_attn_items * hsub
                                : attn_group_count(L.n_attn_items, L.n_trees) * (kAttnGroup / NB);
  const int64_t nblk = L.n_attn_items > 0 ? units * hkv : 0;
  if (nblk == 0) return hipSuccess;
  if (nblk > INT32_MAX) return hipErrorInvalidValue;
  const int32_t n_key_tiles = (int32_t)((L.n_rows + KT - 1) / KT);
  const float sl2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((tree_attn_tiled_kernel<NW, NB>), dim3((unsigned)nblk), dim3(NW * NB * 64), 0, s,
                     reinterpret_cast<const AttnItem *>(L.attn_items), L.n_attn_items, hkv, group, hsub,
                     static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(kt),
                     static_cast<const __bf16 *>(vt), static_cast<__bf16 *>(out), tab, L.row_pos,
                     L.row_trunk_hi, L.row_branch_lo, n_key_tiles, hq, sl2);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const spec_tree_layout &L, int hq, int hkv, const void *q, const void *kws,
                      const void *v, const float2 *tab, float scale, void *out, hipStream_t s) {
  hipLaunchKernelGGL(tree_attn_f32_kernel<D>, dim3((unsigned)L.n_rows, hq), dim3(64), 0, s,
                     static_cast<const float *>(q), static_cast<const float *>(kws),
                     static_cast<const float *>(v), static_cast<float *>(out), tab, L.tree_off,
                     L.row_tree, L.row_pos, L.row_trunk_hi, L.row_branch_lo, L.n_rows, hq, hkv,
                     scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree_attn_tiled(const spec_tree_layout &L, int32_t hq, int32_t hkv, const void *q,
                                  const void *kt, const void *vt, const float2 *tab, float scale,
                                  void *out, hipStream_t s) {
  const int group = hq / hkv;
  if (group >= 8) return launch_tiled<8, 1>(L, hq, hkv, q, kt, vt, tab, scale, out, s);
  if (group >= 3) return launch_tiled<4, 1>(L, hq, hkv, q, kt, vt, tab, scale, out, s);
  if (group == 2) return launch_tiled<2, 2>(L, hq, hkv, q, kt, vt, tab, scale, out, s);
  return launch_tiled<1, 4>(L, hq, hkv, q, kt, vt, tab, scale, out, s);
}

hipError_t launch_tree_attn(const spec_tree_layout &L, int32_t hq, int32_t hkv, int32_t D,
                            spec_dtype dtype, const void *q, const void *kws, const void *v,
                            const float2 *tab, float scale, void *out, hipStream_t s) {
  if (dtype == SPEC_BF16) {
    switch (D) {
      case 32: return launch_bf16_d<32>(L, hq, hkv, q, kws, v, tab, scale, out, s);
      case 64: return launch_bf16_d<64>(L, hq, hkv, q, kws, v, tab, scale, out, s);
      case 128: return launch_bf16_d<128>(L, hq, hkv, q, kws, v, tab, scale, out, s);
    }
  } else {
    switch (D) {
      case 32: return launch_f32<32>(L, hq, hkv, q, kws, v, tab, scale, out, s);
      case 64: return launch_f32<64>(L, hq, hkv, q, kws, v, tab, scale, out, s);
      case 128: return launch_f32<128>(L, hq, hkv, q, kws, v, tab, scale, out, s);
    }
  }
  return hipErrorInvalidValue;
}

// readout[s] = out[pred_row[s]]: one block per step row, 16-byte moves.
__global__ void readout_kernel(const int32_t *__restrict__ pred_row, int64_t row_u4,
                               const uint4 *__restrict__ out, uint4 *__restrict__ readout) {
  const int64_t s = blockIdx.x;
  const uint4 *src = out + (int64_t)pred_row[s] * row_u4;
  uint4 *dst = readout + s * row_u4;
  for (int64_t i = threadIdx.x; i < row_u4; i += blockDim.x) dst[i] = src[i];
}

hipError_t launch_readout(const int32_t *pred_row, int64_t n_steps, int64_t row_bytes,
                          const void *out, void *readout, hipStream_t s) {
  hipLaunchKernelGGL(readout_kernel, dim3((unsigned)n_steps), dim3(256), 0, s, pred_row,
                     row_bytes / 16, static_cast<const uint4 *>(out), static_cast<uint4 *>(readout));
  return hipGetLastError();
}

}  // namespace spec
