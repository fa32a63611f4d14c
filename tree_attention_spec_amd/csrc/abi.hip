// C ABI entry points for attention and E2E-TV: argument checks, workspace
// sizing and dispatch. The pack entry point lives with its kernels.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"

namespace spec {

namespace {
thread_local char g_last_error[512] = {0};
thread_local spec_profile *g_prof = nullptr;
}  // namespace

void prof_mark(hipStream_t s, const char *name) {
  spec_profile *p = g_prof;
  if (!p || p->used >= p->capacity || p->used >= SPEC_PROFILE_MAX) return;
  if (hipEventRecord(static_cast<hipEvent_t>(p->events[p->used]), s) == hipSuccess)
    p->names[p->used++] = name;
}

spec_status fail(spec_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_last_error[0] = 0; }

spec_status hip_fail(hipError_t e, const char *what) {
  return fail(SPEC_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

namespace {

spec_status check_layout(const spec_tree_layout *L, bool need_device) {
  if (!L) return fail(SPEC_ERR_INVALID_ARG, "layout must be non-NULL");
  if (L->n_trees < 1 || L->n_rows < 1 || L->n_steps < 0 || L->n_branches < 0)
    return fail(SPEC_ERR_INVALID_ARG, "layout scalars are not those of a packed tree");
  if (need_device && (!L->tree_off || !L->row_pos || !L->row_trunk_hi || !L->row_branch_lo ||
                      !L->step_off || !L->step_pred_row || !L->attn_items))
    return fail(SPEC_ERR_INVALID_ARG, "layout device arrays are missing (pack with a buffer first)");
  return SPEC_OK;
}

// Workspace of the attention call: RoPE table, then rotated K ([Hkv][N][D]), or,
// for bf16 with head dim 128, rotated K and transposed V in 64-key tiles
// ([Hkv][ceil(N/64)][64*128] each).
struct AttnWork {
  size_t off_tab, off_k, off_v, total;
  bool tiled;
};

AttnWork attn_work(const spec_tree_layout &L, int hkv, int D, spec_dtype dt) {
  AttnWork w{};
  const size_t n_pos = (size_t)L.max_pos + 1;
  w.off_tab = 0;
  w.off_k = align_up(n_pos * (D / 2) * sizeof(float2), 256);
  w.tiled = dt == SPEC_BF16 && D == 128;
  if (w.tiled) {
    const size_t tiles = ((size_t)L.n_rows + kKeyTile - 1) / kKeyTile;
    const size_t bytes = (size_t)hkv * tiles * kKeyTile * D * 2;
    w.off_v = w.off_k + align_up(bytes, 256);
    w.total = w.off_v + align_up(bytes, 256);
  } else {
    const size_t esz = dt == SPEC_BF16 ? 2 : 4;
    w.off_v = 0;
    w.total = align_up(w.off_k + (size_t)L.n_rows * hkv * D * esz, 256);
  }
  return w;
}

}  // namespace

// Workspace of E2E-TV: four float arrays [R], the team partials [R][kTeamMax],
// the team exchange slots [R][kTeamMax], the status and ticket words, the
// per-branch sums [R] (float64; a branch has at least one step), then the
// indicator bitmask [R][bits_row].
static size_t e2etv_bits_row(int64_t V) { return align_up((size_t)(V + 7) / 8, 16); }

namespace {
struct E2etvOffsets {
  size_t step, part, xchg, status, bsum, bits, total;
};
E2etvOffsets e2etv_offsets(int64_t R, int64_t V) {
  E2etvOffsets o;
  o.step = align_up((size_t)R * sizeof(float), 256);
  o.part = 4 * o.step;
  o.xchg = o.part + align_up((size_t)R * kTeamMax * sizeof(float2), 256);
  o.status = o.xchg + align_up((size_t)R * kTeamMax * sizeof(unsigned long long), 256);
  o.bsum = o.status + 256;
  o.bits = o.bsum + align_up((size_t)R * sizeof(double), 256);
  o.total = o.bits + align_up((size_t)R * e2etv_bits_row(V), 256);
  return o;
}
}  // namespace

size_t e2etv_work_bytes(int64_t R, int64_t V) { return e2etv_offsets(R, V).total; }

size_t e2etv_work_bytes_fused(int64_t R) { return e2etv_offsets(R, 8).bits; }

E2etvWork e2etv_carve(void *d_work, int64_t R, int64_t V) {
  char *p = static_cast<char *>(d_work);
  const E2etvOffsets o = e2etv_offsets(R, V);
  E2etvWork w;
  w.lse_q2 = reinterpret_cast<float *>(p);
  w.lse_p2 = reinterpret_cast<float *>(p + o.step);
  w.S = reinterpret_cast<float *>(p + 2 * o.step);
  w.coef = reinterpret_cast<float *>(p + 3 * o.step);
  w.part = reinterpret_cast<float2 *>(p + o.part);
  w.xchg = reinterpret_cast<unsigned long long *>(p + o.xchg);
  w.status = reinterpret_cast<unsigned *>(p + o.status);
  w.branch_sum = reinterpret_cast<double *>(p + o.bsum);
  w.bits = reinterpret_cast<uint8_t *>(p + o.bits);
  w.bits_row = (int64_t)e2etv_bits_row(V);
  return w;
}

}  // namespace spec

using namespace spec;

extern "C" const char *spec_status_string(spec_status s) {
  switch (s) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID_ARG: return "SPEC_ERR_INVALID_ARG";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP";
  }
  return "SPEC_ERR_UNKNOWN";
}

extern "C" const char *spec_last_error(void) { return g_last_error; }

extern "C" int32_t spec_abi_version(void) { return SPEC_TREE_ABI_VERSION; }

extern "C" void spec_profile_attach(spec_profile *p) { g_prof = p; }

extern "C" spec_status spec_tree_attn_fwd(const spec_tree_layout *layout, int32_t hq, int32_t hkv,
                                          int32_t D, spec_dtype dtype, const void *d_q,
                                          const void *d_k, const void *d_v, float rope_base,
                                          float softmax_scale, void *d_out, void *d_readout,
                                          void *d_work, size_t *work_bytes, spec_stream stream) {
  clear_error();
  if (!work_bytes) return fail(SPEC_ERR_INVALID_ARG, "work_bytes must be non-NULL");
  spec_status st = check_layout(layout, d_work != nullptr);
  if (st != SPEC_OK) return st;
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SPEC_ERR_INVALID_ARG, "need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0 (got %d, %d)", hq, hkv);
  if (D != 32 && D != 64 && D != 128)
    return fail(SPEC_ERR_UNSUPPORTED, "head_dim %d not in {32, 64, 128}", D);
  if (dtype != SPEC_BF16 && dtype != SPEC_F32)
    return fail(SPEC_ERR_UNSUPPORTED, "dtype %d not supported", (int)dtype);
  if (dtype == SPEC_BF16 && hq / hkv > 64)
    return fail(SPEC_ERR_UNSUPPORTED, "GQA group %d larger than 64", hq / hkv);
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(SPEC_ERR_INVALID_ARG, "rope_base must be a positive finite number");
  if ((int64_t)layout->n_rows * hq * D > (int64_t)INT32_MAX * 8)
    return fail(SPEC_ERR_UNSUPPORTED, "tensor too large");
  const AttnWork w = attn_work(*layout, hkv, D, dtype);
  // the bf16 kernels address K and V through buffer descriptors whose byte
  // ranges and offsets are 32-bit: all heads' rows for the register-staged
  // kernels, one KV head's 64-key tiles for the tiled kernel
  if (dtype == SPEC_BF16) {
    const int64_t span = w.tiled ? (layout->n_rows + 63) / 64 * 64 * D * 2 : layout->n_rows * hkv * D * 2;
    if (span >= ((int64_t)1 << 32))
      return fail(SPEC_ERR_UNSUPPORTED, "K / V of %lld rows x %d heads x %d dims past the 4 GiB a buffer "
                  "descriptor spans", (long long)layout->n_rows, hkv, D);
  }
  if (!d_work) {
    *work_bytes = w.total;
    return SPEC_OK;
  }
  if (*work_bytes < w.total) {
    size_t have = *work_bytes;
    *work_bytes = w.total;
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, w.total);
  }
  if (!d_q || !d_k || !d_v || !d_out)
    return fail(SPEC_ERR_INVALID_ARG, "d_q, d_k, d_v and d_out must be non-NULL");
  if (!aligned16(d_q) || !aligned16(d_k) || !aligned16(d_v) || !aligned16(d_out) ||
      !aligned16(d_work) || (d_readout && !aligned16(d_readout)))
    return fail(SPEC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *wb = static_cast<char *>(d_work);
  float2 *tab = reinterpret_cast<float2 *>(wb + w.off_tab);
  void *kws = wb + w.off_k;
  prof_mark(s, "attn:begin");
  SPEC_HIP_TRY(launch_rope_table(tab, layout->max_pos + 1, D / 2, (double)rope_base, s));
  prof_mark(s, "rope_table");
  if (w.tiled) {
    void *vws = wb + w.off_v;
    SPEC_HIP_TRY(launch_kv_tiles(d_k, d_v, kws, vws, tab, layout->row_pos, layout->n_rows, hkv, s));
    prof_mark(s, "kv_tiles");
    SPEC_HIP_TRY(launch_tree_attn_tiled(*layout, hq, hkv, d_q, kws, vws, tab, scale, d_out, s));
  } else {
    SPEC_HIP_TRY(launch_rope_k(d_k, kws, tab, layout->row_pos, layout->n_rows, hkv, D, dtype, s));
    prof_mark(s, "rope_k");
    SPEC_HIP_TRY(launch_tree_attn(*layout, hq, hkv, D, dtype, d_q, kws, d_v, tab, scale, d_out, s));
  }
  prof_mark(s, "tree_attn");
  if (d_readout && layout->n_steps > 0) {
    const int64_t row_bytes = (int64_t)hq * D * (dtype == SPEC_BF16 ? 2 : 4);
    SPEC_HIP_TRY(launch_readout(layout->step_pred_row, layout->n_steps, row_bytes, d_out,
                                d_readout, s));
    prof_mark(s, "readout");
  }
  return SPEC_OK;
}

namespace {
// Checks of spec_e2etv_fwd_bwd that need no buffer: the layout, vocabulary, dtype
// and normaliser.
spec_status check_e2etv_shape(const spec_tree_layout *layout, int64_t vocab, spec_dtype dtype,
                              float inv_norm, bool need_device) {
  if (!layout) return fail(SPEC_ERR_INVALID_ARG, "layout must be non-NULL");
  if (layout->n_steps < 1 || layout->n_branches < 1)
    return fail(SPEC_ERR_INVALID_ARG, "the layout has no supervised steps");
  if (need_device && (!layout->step_off || !layout->step_branch))
    return fail(SPEC_ERR_INVALID_ARG, "layout device arrays are missing (pack with a buffer first)");
  if (vocab < 1 || vocab > (int64_t)INT32_MAX)
    return fail(SPEC_ERR_INVALID_ARG, "vocab %lld out of range", (long long)vocab);
  if (dtype != SPEC_BF16 && dtype != SPEC_F32)
    return fail(SPEC_ERR_UNSUPPORTED, "logit dtype %d not supported", (int)dtype);
  if (!std::isfinite(inv_norm)) return fail(SPEC_ERR_INVALID_ARG, "inv_norm must be finite");
  return SPEC_OK;
}

spec_status check_e2etv_buffers(const void *d_draft, const void *d_teacher, const float *d_alpha,
                                const float *d_loss, const float *d_grad) {
  if (!d_draft || !d_teacher || !d_alpha || !d_loss)
    return fail(SPEC_ERR_INVALID_ARG, "d_draft, d_teacher, d_alpha and d_loss must be non-NULL");
  if (!aligned16(d_draft) || !aligned16(d_teacher) || (d_grad && !aligned16(d_grad)))
    return fail(SPEC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  return SPEC_OK;
}
}  // namespace

extern "C" spec_status spec_e2etv_fwd_bwd(const spec_tree_layout *layout, int64_t vocab,
                                          spec_dtype dtype, const void *d_draft,
                                          const void *d_teacher, float inv_norm, float *d_alpha,
                                          float *d_loss, float *d_grad, void *d_work,
                                          size_t *work_bytes, spec_stream stream) {
  clear_error();
  if (!work_bytes) return fail(SPEC_ERR_INVALID_ARG, "work_bytes must be non-NULL");
  spec_status st = check_e2etv_shape(layout, vocab, dtype, inv_norm, d_work != nullptr);
  if (st != SPEC_OK) return st;
  const size_t need = e2etv_work_bytes(layout->n_steps, vocab);
  if (!d_work) {
    *work_bytes = need;
    return SPEC_OK;
  }
  if (*work_bytes < need) {
    size_t have = *work_bytes;
    *work_bytes = need;
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  }
  st = check_e2etv_buffers(d_draft, d_teacher, d_alpha, d_loss, d_grad);
  if (st != SPEC_OK) return st;
  if (!aligned16(d_work)) return fail(SPEC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  const float w = inv_norm > 0.f ? inv_norm : (float)(1.0 / (double)layout->n_steps);
  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_mark(s, "e2etv:begin");
  SPEC_HIP_TRY(launch_e2etv(*layout, vocab, dtype, d_draft, d_teacher, w, d_alpha, d_loss, d_grad,
                            e2etv_carve(d_work, layout->n_steps, vocab), s));
  return SPEC_OK;
}

extern "C" spec_status spec_qsa_attn_fwd(const spec_tree_layout *layout, int32_t hq, int32_t hkv, int32_t D,
                                         int32_t index_dim, int32_t group_size, int32_t top_k,
                                         const void *d_q, const void *d_k, const void *d_v, const void *d_qi,
                                         const void *d_ki, float rope_base, float softmax_scale, void *d_out,
                                         int32_t *d_selected, void *d_readout, void *d_work,
                                         size_t *work_bytes, spec_stream stream) {
  clear_error();
  if (!work_bytes) return fail(SPEC_ERR_INVALID_ARG, "work_bytes must be non-NULL");
  spec_status st = check_layout(layout, d_work != nullptr);
  if (st != SPEC_OK) return st;
  if (d_work && (!layout->row_tree || !layout->row_branch || !layout->row_anchor || !layout->branch_tree ||
                 !layout->branch_anchor || !layout->branch_len || !layout->branch_off || !layout->tree_trunk_len))
    return fail(SPEC_ERR_INVALID_ARG, "layout device arrays are missing (pack with a buffer first)");
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(SPEC_ERR_INVALID_ARG, "need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0 (got %d, %d)", hq, hkv);
  if (D != 128) return fail(SPEC_ERR_UNSUPPORTED, "head_dim %d: the sparse path takes 128", D);
  if (hq / hkv > 16) return fail(SPEC_ERR_UNSUPPORTED, "GQA group %d larger than 16", hq / hkv);
  if (index_dim < 8 || index_dim > 256 || index_dim % 8 != 0)
    return fail(SPEC_ERR_UNSUPPORTED, "index_dim %d: a multiple of 8 in [8, 256]", index_dim);
  if (group_size < 1 || top_k < 1 || top_k > 64)
    return fail(SPEC_ERR_INVALID_ARG, "need group_size >= 1 and 1 <= top_k <= 64 (got %d, %d)", group_size,
                top_k);
  if (((int64_t)layout->max_pos + 1) / group_size > 1024)
    return fail(SPEC_ERR_UNSUPPORTED, "%lld complete groups per row (at most 1024)",
                (long long)(((int64_t)layout->max_pos + 1) / group_size));
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(SPEC_ERR_INVALID_ARG, "rope_base must be a positive finite number");
  const int64_t n_tiles = (layout->n_rows + kKeyTile - 1) / kKeyTile;
  if (n_tiles * kKeyTile * D * 2 >= ((int64_t)1 << 31) || (int64_t)layout->n_rows * hq * D >= ((int64_t)1 << 31))
    return fail(SPEC_ERR_UNSUPPORTED, "tensor too large for 32-bit offsets");
  const AttnWork w = attn_work(*layout, hkv, D, SPEC_BF16);
  const size_t off_keys = w.total;
  const size_t off_sel = off_keys + align_up(qsa_keys_floats(*layout, hkv, index_dim, group_size) * 4, 256);
  const size_t total = off_sel + align_up((size_t)layout->n_rows * hkv * top_k * 4, 256);
  if (!d_work) {
    *work_bytes = total;
    return SPEC_OK;
  }
  if (*work_bytes < total) {
    size_t have = *work_bytes;
    *work_bytes = total;
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, total);
  }
  if (!d_q || !d_k || !d_v || !d_qi || !d_ki || !d_out)
    return fail(SPEC_ERR_INVALID_ARG, "d_q, d_k, d_v, d_qi, d_ki and d_out must be non-NULL");
  if (!aligned16(d_q) || !aligned16(d_k) || !aligned16(d_v) || !aligned16(d_qi) || !aligned16(d_ki) ||
      !aligned16(d_out) || !aligned16(d_work) || (d_readout && !aligned16(d_readout)) ||
      (d_selected && !aligned16(d_selected)))
    return fail(SPEC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *wb = static_cast<char *>(d_work);
  float2 *tab = reinterpret_cast<float2 *>(wb + w.off_tab);
  prof_mark(s, "qsa:begin");
  SPEC_HIP_TRY(launch_rope_table(tab, layout->max_pos + 1, D / 2, (double)rope_base, s));
  prof_mark(s, "rope_table");
  SPEC_HIP_TRY(launch_kv_tiles(d_k, d_v, wb + w.off_k, wb + w.off_v, tab, layout->row_pos, layout->n_rows, hkv, s));
  prof_mark(s, "kv_tiles");
  int32_t *sel = d_selected ? d_selected : reinterpret_cast<int32_t *>(wb + off_sel);
  SPEC_HIP_TRY(launch_qsa(*layout, hq, hkv, index_dim, group_size, top_k, d_q, d_qi, d_ki, wb + w.off_k,
                          wb + w.off_v, tab, scale, reinterpret_cast<float *>(wb + off_keys), sel, d_out, s));
  if (d_readout && layout->n_steps > 0) {
    SPEC_HIP_TRY(launch_readout(layout->step_pred_row, layout->n_steps, (int64_t)hq * D * 2, d_out, d_readout, s));
    prof_mark(s, "readout");
  }
  return SPEC_OK;
}

// ---------------------------------------------------------------- no-allocation E2E-TV
// The workspace of spec_e2etv_fwd_bwd_noalloc: one array per device, held by the
// loaded code object until the process ends. Its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and only that address
// is handed to kernels: in host code `scratch` names a host-side stand-in.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

spec_status scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SPEC_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned16(p)) return fail(SPEC_ERR_HIP, "scratch has no usable device address");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SPEC_OK;
}
}  // namespace

extern "C" spec_status spec_e2etv_fwd_bwd_noalloc(const spec_tree_layout *layout, int64_t vocab,
                                                  spec_dtype dtype, const void *d_draft,
                                                  const void *d_teacher, float inv_norm,
                                                  float *d_alpha, float *d_loss, float *d_grad,
                                                  spec_stream stream) {
  clear_error();
  spec_status st = check_e2etv_shape(layout, vocab, dtype, inv_norm, true);
  if (st != SPEC_OK) return st;
  st = check_e2etv_buffers(d_draft, d_teacher, d_alpha, d_loss, d_grad);
  if (st != SPEC_OK) return st;
  const int64_t R = layout->n_steps;
  const size_t cap = SPEC_NOALLOC_SCRATCH_BYTES;
  const size_t need = e2etv_work_bytes(R, vocab);
  bool with_bits = need <= cap;
  if (!with_bits) {
    // the fused pipeline needs no bitmask; every other path does
    bool fused = false;
    if (dtype == SPEC_BF16 && vocab % 8 == 0 && e2etv_work_bytes_fused(R) <= cap)
      SPEC_HIP_TRY(e2etv_takes_fused_path(*layout, vocab, dtype, &fused));
    if (!fused)
      return fail(SPEC_ERR_UNSUPPORTED,
                  "%lld steps x vocabulary %lld need %zu bytes of scratch; the no-allocation entry "
                  "point holds %zu (use spec_e2etv_fwd_bwd with a workspace)",
                  (long long)R, (long long)vocab, fused ? e2etv_work_bytes_fused(R) : need, cap);
  }
  void *base = nullptr;
  st = scratch_address(&base);
  if (st != SPEC_OK) return st;
  E2etvWork ws = e2etv_carve(base, R, vocab);
  if (!with_bits) ws.bits = nullptr;
  const float w = inv_norm > 0.f ? inv_norm : (float)(1.0 / (double)R);
  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_mark(s, "e2etv:begin");
  SPEC_HIP_TRY(launch_e2etv(*layout, vocab, dtype, d_draft, d_teacher, w, d_alpha, d_loss, d_grad, ws, s));
  return SPEC_OK;
}

extern "C" spec_status spec_e2etv_status(const spec_tree_layout *layout, int64_t vocab, const void *d_work,
                                         uint32_t *h_status, spec_stream stream) {
  clear_error();
  if (!layout || !h_status) return fail(SPEC_ERR_INVALID_ARG, "layout and h_status must be non-NULL");
  if (layout->n_steps < 1) return fail(SPEC_ERR_INVALID_ARG, "the layout has no supervised steps");
  if (vocab < 1 || vocab > (int64_t)INT32_MAX)
    return fail(SPEC_ERR_INVALID_ARG, "vocab %lld out of range", (long long)vocab);
  const void *base = d_work;
  if (!base) {
    void *p = nullptr;
    spec_status st = scratch_address(&p);
    if (st != SPEC_OK) return st;
    base = p;
  }
  const E2etvWork w = e2etv_carve(const_cast<void *>(base), layout->n_steps, vocab);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  SPEC_HIP_TRY(hipMemcpyAsync(&v, w.status, sizeof(v), hipMemcpyDeviceToHost, s));
  SPEC_HIP_TRY(hipStreamSynchronize(s));
  *h_status = v;
  return SPEC_OK;
}

extern "C" spec_status spec_e2etv_head_fwd_bwd(const spec_tree_layout *layout, int64_t vocab,
                                               int32_t d_model, spec_dtype dtype,
                                               const void *d_draft, const void *d_hidden,
                                               const void *d_head, float inv_norm, float *d_alpha,
                                               float *d_loss, float *d_grad, void *d_work,
                                               size_t *work_bytes, spec_stream stream) {
  clear_error();
  if (!work_bytes) return fail(SPEC_ERR_INVALID_ARG, "work_bytes must be non-NULL");
  if (!layout) return fail(SPEC_ERR_INVALID_ARG, "layout must be non-NULL");
  if (layout->n_steps < 1 || layout->n_branches < 1)
    return fail(SPEC_ERR_INVALID_ARG, "the layout has no supervised steps");
  if (d_work && (!layout->step_off || !layout->step_pred_row))
    return fail(SPEC_ERR_INVALID_ARG, "layout device arrays are missing (pack with a buffer first)");
  if (vocab < 1 || vocab > (int64_t)INT32_MAX)
    return fail(SPEC_ERR_INVALID_ARG, "vocab %lld out of range", (long long)vocab);
  if (d_model < 1) return fail(SPEC_ERR_INVALID_ARG, "d_model %d out of range", (int)d_model);
  if (vocab % 8 != 0 || d_model % 64 != 0)
    return fail(SPEC_ERR_UNSUPPORTED, "vocab (%lld) must be a multiple of 8 and d_model (%d) of 64",
                (long long)vocab, (int)d_model);
  // the head kernels address the hidden states, and each 256-row tile of the
  // head, through buffer descriptors
  if ((uint64_t)layout->n_rows * (uint64_t)d_model * 2u > (uint64_t)INT32_MAX || d_model > (1 << 22))
    return fail(SPEC_ERR_UNSUPPORTED, "hidden states of %lld rows x %d exceed 2 GiB, or d_model past 2^22",
                (long long)layout->n_rows, (int)d_model);
  if (layout->max_branch_len > 64)
    return fail(SPEC_ERR_UNSUPPORTED, "branches of %d steps (at most 64)", (int)layout->max_branch_len);
  if (dtype != SPEC_BF16 && dtype != SPEC_F32)
    return fail(SPEC_ERR_UNSUPPORTED, "draft dtype %d not supported", (int)dtype);
  if (!std::isfinite(inv_norm)) return fail(SPEC_ERR_INVALID_ARG, "inv_norm must be finite");
  const size_t need = e2etv_head_work_bytes(layout->n_steps, vocab);
  if (!d_work) {
    *work_bytes = need;
    return SPEC_OK;
  }
  if (*work_bytes < need) {
    size_t have = *work_bytes;
    *work_bytes = need;
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  }
  if (!d_draft || !d_hidden || !d_head || !d_alpha || !d_loss)
    return fail(SPEC_ERR_INVALID_ARG,
                "d_draft, d_hidden, d_head, d_alpha and d_loss must be non-NULL");
  if (!aligned16(d_draft) || !aligned16(d_hidden) || !aligned16(d_head) || !aligned16(d_work) ||
      (d_grad && !aligned16(d_grad)))
    return fail(SPEC_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  const float w = inv_norm > 0.f ? inv_norm : (float)(1.0 / (double)layout->n_steps);
  hipStream_t s = static_cast<hipStream_t>(stream);
  prof_mark(s, "e2etv_head:begin");
  SPEC_HIP_TRY(launch_e2etv_head(*layout, vocab, d_model, dtype, d_draft, d_hidden, d_head, w,
                                 d_alpha, d_loss, d_grad, d_work, s));
  return SPEC_OK;
}
