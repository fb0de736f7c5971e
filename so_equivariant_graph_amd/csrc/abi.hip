// C-ABI entry points: argument validation on the host, workspace carving and
// kernel dispatch.  Every argument error is returned before any launch.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "common.h"
#include "launch.h"
#include "norm.h"
#include "swiglu.h"
#include "wigner.h"

namespace so2 {

static thread_local char g_last_error[256] = "";

so2_status device_error(hipError_t err) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(err),
           hipGetErrorString(err));
  return SO2_ERR_DEVICE;
}

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

enum Kind { kNone = 0, kValu = 1, kMfma = 2, kBatch = 3 };

so2_status check_desc(const so2_attn_desc* d) {
  if (!d) return SO2_ERR_INVALID_ARGUMENT;
  if (d->n_atoms < 1 || d->n_targets < 0 || d->n_targets > d->n_atoms) return SO2_ERR_INVALID_ARGUMENT;
  if (d->l_max < 0 || d->channels < 1 || d->heads < 1) return SO2_ERR_INVALID_ARGUMENT;
  if (d->channels % d->heads) return SO2_ERR_INVALID_ARGUMENT;
  if (d->n_rbf < 2 || d->envelope_p < 1 || d->envelope_p > 64) return SO2_ERR_INVALID_ARGUMENT;
  if (!(d->cutoff > 0.0f) || !isfinite(d->cutoff)) return SO2_ERR_INVALID_ARGUMENT;
  if (d->flags & ~(uint32_t)(SO2_FLAG_RBF_ENVELOPE | SO2_FLAG_NO_RADIAL)) return SO2_ERR_INVALID_ARGUMENT;
  if (d->dtype != SO2_FP32 && d->dtype != SO2_BF16) return SO2_ERR_INVALID_ARGUMENT;
  if (d->l_max > kMaxL) return SO2_ERR_UNSUPPORTED;
  return SO2_OK;
}

// The base layer: every order, one stream (the radial logit bias is carried
// by both kernels).
const so2_attn_variant kBase = {-1, 1};

so2_status check_variant(const so2_attn_desc* d, const so2_attn_variant* v) {
  if (!v) return SO2_ERR_INVALID_ARGUMENT;
  if (v->m_max < -1 || v->m_max > d->l_max) return SO2_ERR_INVALID_ARGUMENT;
  if (v->n_focus < 1 || d->channels % v->n_focus) return SO2_ERR_INVALID_ARGUMENT;
  return SO2_OK;
}

bool is_base(const so2_attn_desc* d, const so2_attn_variant* v) {
  return (v->m_max < 0 || v->m_max == d->l_max) && v->n_focus == 1;
}

// bf16 shapes the MFMA kernel takes run there: the base layer, truncated
// orders (m_max < L), and 2, 4 or 8 focus streams at L <= 4 with every
// order and whole heads per stream; past its size limit they are refused
// (kNone) rather than moved to a slower path.  Everything else (fp32, other
// shapes, other focus streams) runs on the fp32 edge-batch path, which
// reads the edge count back once; with allow_wait false (callers that must
// not wait on the stream) it runs on the fp32 VALU kernel instead, which
// takes the base layer only.
Kind pick_kind(const so2_attn_desc* d, const so2_attn_variant* v = &kBase, bool allow_wait = true) {
  const int mm = v->m_max < 0 ? d->l_max : v->m_max;
  if (d->dtype == SO2_BF16 && mfma_shape(d->l_max, d->channels, d->heads, d->n_rbf) &&
      mfma_focus(d->l_max, d->heads, mm, v->n_focus))
    return mfma_fits(d->l_max, d->n_atoms) ? kMfma : kNone;
  if (allow_wait && batch_fwd_supported(d->l_max, d->channels, d->heads, d->n_rbf, mm, v->n_focus)) return kBatch;
  if (!allow_wait && is_base(d, v) && valu_supported(d->l_max, d->channels, d->heads)) return kValu;
  return kNone;
}

struct AttnLayout {
  size_t q, k, scratch, scratch_bytes, total;
};

AttnLayout attn_layout(const so2_attn_desc* d, Kind kind, const so2_attn_variant* v = &kBase) {
  AttnLayout L{};
  size_t off = 0;
  L.q = off;
  off += align256(sizeof(float) * (size_t)d->n_targets * d->channels);
  L.k = off;
  off += align256(sizeof(float) * (size_t)d->n_atoms * d->channels);
  L.scratch = off;
  const int mm = v->m_max < 0 ? d->l_max : v->m_max;
  L.scratch_bytes = kind == kMfma    ? mfma_scratch_bytes(d->n_atoms, d->n_targets, d->l_max, d->heads, d->n_rbf)
                    : kind == kBatch ? batch_fwd_scratch_bytes(d->n_targets, d->l_max, d->channels, d->heads, mm, v->n_focus)
                                     : valu_scratch_bytes(d->l_max, d->channels);
  off += align256(L.scratch_bytes);
  L.total = off;
  return L;
}

so2_status check_box(const float* box_host, float cutoff) {
  if (!box_host) return SO2_OK;
  for (int d = 0; d < 3; ++d) {
    if (!isfinite(box_host[d]) || !(box_host[d] > 0.0f)) return SO2_ERR_INVALID_ARGUMENT;
    if (!((double)box_host[d] > 2.0 * (double)cutoff)) return SO2_ERR_BOX;
  }
  return SO2_OK;
}

}  // namespace
}  // namespace so2

using namespace so2;

extern "C" {

const char* so2_status_string(so2_status s) {
  switch (s) {
    case SO2_OK:
      return "SO2_OK";
    case SO2_ERR_INVALID_ARGUMENT:
      return "SO2_ERR_INVALID_ARGUMENT";
    case SO2_ERR_UNSUPPORTED:
      return "SO2_ERR_UNSUPPORTED";
    case SO2_ERR_CAPACITY:
      return "SO2_ERR_CAPACITY";
    case SO2_ERR_BOX:
      return "SO2_ERR_BOX";
    case SO2_ERR_DEVICE:
      return "SO2_ERR_DEVICE";
    case SO2_ERR_WORKSPACE:
      return "SO2_ERR_WORKSPACE";
  }
  return "SO2_ERR_UNKNOWN";
}

const char* so2_last_device_error(void) { return g_last_error; }

size_t so2_neighbors_workspace_bytes(int32_t n_atoms) { return neighbors_workspace_bytes(n_atoms); }

so2_status build_neighbors(const float* pos, int32_t n_atoms, const int32_t* mol_id,
                           const float* box_host, float cutoff, int32_t* row_ptr, int32_t* col,
                           int64_t capacity, int64_t* n_edges_host, void* workspace,
                           size_t workspace_bytes, so2_stream_t stream) {
  if (!pos || !row_ptr || !n_edges_host || !workspace) return SO2_ERR_INVALID_ARGUMENT;
  if (n_atoms < 1 || capacity < 0) return SO2_ERR_INVALID_ARGUMENT;
  if (!col && capacity > 0) return SO2_ERR_INVALID_ARGUMENT;
  if (!(cutoff > 0.0f) || !isfinite(cutoff)) return SO2_ERR_INVALID_ARGUMENT;
  so2_status st = check_box(box_host, cutoff);
  if (st != SO2_OK) return st;
  return neighbors_build(pos, n_atoms, mol_id, box_host, cutoff, row_ptr, col, capacity,
                         n_edges_host, workspace, workspace_bytes, (hipStream_t)stream);
}

int64_t so2_weight_count(int32_t l_max, int32_t channels) {
  if (l_max < 0 || channels < 1) return -1;
  const int64_t L = l_max, C = channels;
  return C * C * ((L + 1) * (L + 1) + L * (L + 1) * (2 * L + 1) / 3);
}

int64_t so2_weight_count_variant(int32_t l_max, int32_t channels, int32_t m_max, int32_t n_focus) {
  if (l_max < 0 || channels < 1 || n_focus < 1 || channels % n_focus) return -1;
  if (m_max < 0) m_max = l_max;
  if (m_max > l_max) return -1;
  return (int64_t)n_focus * so2_w1_offset(l_max, channels / n_focus, m_max + 1);
}

size_t so2_attention_workspace_bytes(const so2_attn_desc* desc) {
  if (check_desc(desc) != SO2_OK) return 0;
  Kind kind = pick_kind(desc);
  if (kind == kNone) return 0;
  return attn_layout(desc, kind).total;
}

int32_t so2_attention_kernel_kind(const so2_attn_desc* desc) {
  if (check_desc(desc) != SO2_OK) return 0;
  return (int32_t)pick_kind(desc);
}

static so2_status attention_fwd_impl(uint32_t stages, const so2_attn_desc* desc, const so2_attn_variant* var,
                                     const float* pos, const float* box_host, const int32_t* row_ptr,
                                     const int32_t* col, const void* x, const void* w_q, const void* w_k,
                                     const void* w_rad, const void* w_so2, const void* w_logit, const void* w_focus,
                                     float* y, void* workspace, size_t workspace_bytes, so2_stream_t stream,
                                     bool allow_wait = true) {
  if (stages == 0 || (stages & ~(uint32_t)(SO2_STAGE_PREPARE | SO2_STAGE_FUSED))) return SO2_ERR_INVALID_ARGUMENT;
  so2_status st = check_desc(desc);
  if (st != SO2_OK) return st;
  st = check_variant(desc, var);
  if (st != SO2_OK) return st;
  if (var->n_focus > 1 && !w_focus) return SO2_ERR_INVALID_ARGUMENT;
  Kind kind = pick_kind(desc, var, allow_wait);
  if (kind == kNone) return SO2_ERR_UNSUPPORTED;
  st = check_box(box_host, desc->cutoff);
  if (st != SO2_OK) return st;
  if (!pos || !row_ptr || !col || !x || !w_q || !w_k || !w_rad || !w_so2 || !workspace)
    return SO2_ERR_INVALID_ARGUMENT;
  if ((stages & SO2_STAGE_FUSED) && !y) return SO2_ERR_INVALID_ARGUMENT;
  const AttnLayout lay = attn_layout(desc, kind, var);
  if (workspace_bytes < lay.total || ((uintptr_t)workspace & 255)) return SO2_ERR_WORKSPACE;

  AttnArgs a{};
  a.pos = pos;
  a.row_ptr = row_ptr;
  a.col = col;
  a.x = x;
  a.w_q = w_q;
  a.w_k = w_k;
  a.w_rad = w_rad;
  a.w_so2 = w_so2;
  a.y = y;
  char* ws = (char*)workspace;
  a.q = (float*)(ws + lay.q);
  a.k = (float*)(ws + lay.k);
  a.scratch = ws + lay.scratch;
  a.scratch_bytes = lay.scratch_bytes;
  a.n_atoms = desc->n_atoms;
  a.n_targets = desc->n_targets;
  a.L = desc->l_max;
  a.C = desc->channels;
  a.H = desc->heads;
  a.K = desc->n_rbf;
  a.p = desc->envelope_p;
  a.cutoff = desc->cutoff;
  a.flags = desc->flags;
  a.dtype = desc->dtype;
  a.periodic = box_host != nullptr;
  for (int d = 0; d < 3; ++d) a.box[d] = box_host ? box_host[d] : 0.0f;
  a.m_max = var->m_max < 0 ? desc->l_max : var->m_max;
  a.n_focus = var->n_focus;
  a.w_logit = w_logit;
  a.w_focus = w_focus;

  if (kind == kMfma && !mfma_aligned(a)) return SO2_ERR_INVALID_ARGUMENT;

  hipStream_t s = (hipStream_t)stream;
  if (stages & SO2_STAGE_PREPARE) {
    st = launch_qk_proj(a, s);
    if (st != SO2_OK) return st;
    if (kind == kMfma) {
      st = launch_attention_mfma_prep(a, s);
      if (st != SO2_OK) return st;
    }
  }
  if (stages & SO2_STAGE_FUSED) {
    st = kind == kMfma ? launch_attention_mfma(a, s)
         : kind == kBatch ? launch_attention_batch_fwd(a, s)
                          : launch_attention_valu(a, s);
    if (st != SO2_OK) return st;
  }
  return SO2_OK;
}

static so2_status bwd_layout(const so2_attn_desc* d, AttnLayout* out) {
  so2_status st = check_desc(d);
  if (st != SO2_OK) return st;
  if (!bwd_supported(d->l_max, d->channels, d->heads, d->n_rbf)) return SO2_ERR_UNSUPPORTED;
  AttnLayout L{};
  size_t off = 0;
  L.q = off;
  off += align256(sizeof(float) * (size_t)d->n_atoms * d->channels);
  L.k = off;
  off += align256(sizeof(float) * (size_t)d->n_atoms * d->channels);
  L.scratch = off;
  L.scratch_bytes = bwd_scratch_bytes(d->n_atoms, d->n_targets, d->l_max, d->channels, d->heads, d->n_rbf);
  off += align256(L.scratch_bytes);
  L.total = off;
  *out = L;
  return SO2_OK;
}

size_t so2_attention_bwd_workspace_bytes(const so2_attn_desc* desc) {
  AttnLayout L{};
  return bwd_layout(desc, &L) == SO2_OK ? L.total : 0;
}

so2_status so2_attention_bwd(const so2_attn_desc* desc, const float* pos, const float* box_host,
                             const int32_t* row_ptr, const int32_t* col, const void* x, const void* w_q,
                             const void* w_k, const void* w_rad, const void* w_so2, const float* dy, float* dx,
                             float* dpos, float* dw_q, float* dw_k, float* dw_rad, float* dw_so2, void* workspace,
                             size_t workspace_bytes, so2_stream_t stream) {
  AttnLayout lay{};
  so2_status st = bwd_layout(desc, &lay);
  if (st != SO2_OK) return st;
  st = check_box(box_host, desc->cutoff);
  if (st != SO2_OK) return st;
  if (!pos || !row_ptr || !col || !x || !w_q || !w_k || !w_rad || !w_so2 || !dy || !dx || !dpos || !workspace)
    return SO2_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < lay.total || ((uintptr_t)workspace & 255)) return SO2_ERR_WORKSPACE;
  AttnArgs a{};
  a.pos = pos;
  a.row_ptr = row_ptr;
  a.col = col;
  a.x = x;
  a.w_q = w_q;
  a.w_k = w_k;
  a.w_rad = w_rad;
  a.w_so2 = w_so2;
  char* ws = (char*)workspace;
  a.q = (float*)(ws + lay.q);
  a.k = (float*)(ws + lay.k);
  a.scratch = ws + lay.scratch;
  a.scratch_bytes = lay.scratch_bytes;
  a.n_atoms = desc->n_atoms;
  a.n_targets = desc->n_atoms;  // q for every atom (the projection kernel's row count)
  a.L = desc->l_max;
  a.C = desc->channels;
  a.H = desc->heads;
  a.K = desc->n_rbf;
  a.p = desc->envelope_p;
  a.cutoff = desc->cutoff;
  a.flags = desc->flags;
  a.dtype = desc->dtype;
  a.periodic = box_host != nullptr;
  for (int d = 0; d < 3; ++d) a.box[d] = box_host ? box_host[d] : 0.0f;
  a.m_max = desc->l_max;
  a.n_focus = 1;
  hipStream_t s = (hipStream_t)stream;
  st = launch_qk_proj(a, s);
  if (st != SO2_OK) return st;
  a.n_targets = desc->n_targets;
  return launch_attention_bwd(a, dy, dx, dpos, dw_q, dw_k, dw_rad, dw_so2, s);
}

so2_status so2_attention_fwd_stages(uint32_t stages, const so2_attn_desc* desc, const float* pos,
                                    const float* box_host, const int32_t* row_ptr, const int32_t* col,
                                    const void* x, const void* w_q, const void* w_k, const void* w_rad,
                                    const void* w_so2, float* y, void* workspace, size_t workspace_bytes,
                                    so2_stream_t stream) {
  return attention_fwd_impl(stages, desc, &kBase, pos, box_host, row_ptr, col, x, w_q, w_k, w_rad, w_so2, nullptr,
                            nullptr, y, workspace, workspace_bytes, stream);
}

so2_status so2_attention_fwd(const so2_attn_desc* desc, const float* pos, const float* box_host,
                             const int32_t* row_ptr, const int32_t* col, const void* x,
                             const void* w_q, const void* w_k, const void* w_rad,
                             const void* w_so2, float* y, void* workspace,
                             size_t workspace_bytes, so2_stream_t stream) {
  return so2_attention_fwd_stages(SO2_STAGE_PREPARE | SO2_STAGE_FUSED, desc, pos, box_host, row_ptr, col, x, w_q,
                                  w_k, w_rad, w_so2, y, workspace, workspace_bytes, stream);
}

size_t so2_attention_variant_workspace_bytes(const so2_attn_desc* desc, const so2_attn_variant* var) {
  if (check_desc(desc) != SO2_OK || check_variant(desc, var) != SO2_OK) return 0;
  Kind kind = pick_kind(desc, var);
  if (kind == kNone) return 0;
  return attn_layout(desc, kind, var).total;
}

int32_t so2_attention_variant_kernel_kind(const so2_attn_desc* desc, const so2_attn_variant* var) {
  if (check_desc(desc) != SO2_OK || check_variant(desc, var) != SO2_OK) return 0;
  return (int32_t)pick_kind(desc, var);
}

so2_status so2_attention_fwd_variant(const so2_attn_desc* desc, const so2_attn_variant* var, const float* pos,
                                     const float* box_host, const int32_t* row_ptr, const int32_t* col,
                                     const void* x, const void* w_q, const void* w_k, const void* w_rad,
                                     const void* w_so2, const void* w_logit, const void* w_focus, float* y,
                                     void* workspace, size_t workspace_bytes, so2_stream_t stream) {
  return attention_fwd_impl(SO2_STAGE_PREPARE | SO2_STAGE_FUSED, desc, var, pos, box_host, row_ptr, col, x, w_q,
                            w_k, w_rad, w_so2, w_logit, w_focus, y, workspace, workspace_bytes, stream);
}

so2_status so2_merged_rms_norm(const void* x, const float* gamma, void* y, int32_t n_atoms, int32_t l_max,
                               int32_t channels, float eps, int32_t dtype, so2_stream_t stream) {
  if (n_atoms < 0 || l_max < 0 || channels < 1 || !(eps >= 0.0f) || !isfinite(eps)) return SO2_ERR_INVALID_ARGUMENT;
  if (dtype != SO2_FP32 && dtype != SO2_BF16) return SO2_ERR_INVALID_ARGUMENT;
  if (n_atoms > 0 && (!x || !gamma || !y)) return SO2_ERR_INVALID_ARGUMENT;
  if (l_max > kMaxL) return SO2_ERR_UNSUPPORTED;
  return launch_merged_rms_norm(x, gamma, y, n_atoms, l_max, channels, eps, dtype, (hipStream_t)stream);
}

size_t so2_swiglu_s2_workspace_bytes(int32_t n_atoms, int32_t l_max, int32_t channels, int32_t dtype) {
  if (n_atoms < 0 || l_max < 0 || l_max > kMaxL || channels < 1) return 0;
  if (dtype != SO2_FP32 && dtype != SO2_BF16) return 0;
  return swiglu_s2_workspace_bytes(n_atoms, l_max, channels, dtype);
}

so2_status so2_swiglu_s2_stages(uint32_t stages, const void* x, const void* w_a, const void* w_b, const void* w_g,
                                const void* w_o, float* y, int32_t n_atoms, int32_t l_max, int32_t channels,
                                int32_t dtype, void* workspace, size_t workspace_bytes, so2_stream_t stream) {
  if (stages == 0 || (stages & ~(uint32_t)(SO2_STAGE_SW_MAPS | SO2_STAGE_SW_GRID | SO2_STAGE_SW_OUT)))
    return SO2_ERR_INVALID_ARGUMENT;
  if (n_atoms < 0 || l_max < 0 || channels < 1) return SO2_ERR_INVALID_ARGUMENT;
  if (dtype != SO2_FP32 && dtype != SO2_BF16) return SO2_ERR_INVALID_ARGUMENT;
  if (n_atoms > 0 && (!x || !w_a || !w_b || !w_g || !w_o || !y)) return SO2_ERR_INVALID_ARGUMENT;
  if (l_max > kMaxL) return SO2_ERR_UNSUPPORTED;
  return launch_swiglu_s2(stages, x, w_a, w_b, w_g, w_o, y, n_atoms, l_max, channels, dtype, workspace,
                          workspace_bytes, (hipStream_t)stream);
}

so2_status so2_swiglu_s2(const void* x, const void* w_a, const void* w_b, const void* w_g, const void* w_o, float* y,
                         int32_t n_atoms, int32_t l_max, int32_t channels, int32_t dtype, void* workspace,
                         size_t workspace_bytes, so2_stream_t stream) {
  return so2_swiglu_s2_stages(SO2_STAGE_SW_MAPS | SO2_STAGE_SW_GRID | SO2_STAGE_SW_OUT, x, w_a, w_b, w_g, w_o, y,
                              n_atoms, l_max, channels, dtype, workspace, workspace_bytes, stream);
}

so2_status so2_edge_frame_host(int32_t l_max, const float* rhat, float* R_out, float* D_out) {
  if (!rhat || !R_out || !D_out || l_max < 0 || l_max > kMaxL) return SO2_ERR_INVALID_ARGUMENT;
  float n = sqrtf(rhat[0] * rhat[0] + rhat[1] * rhat[1] + rhat[2] * rhat[2]);
  if (!(n > 0.0f) || !isfinite(n)) return SO2_ERR_INVALID_ARGUMENT;
  edge_frame(rhat[0] / n, rhat[1] / n, rhat[2] / n, R_out);
  wigner_blocks_serial(l_max, R_out, D_out);
  return SO2_OK;
}

so2_status so2_wigner_generators_host(int32_t l_max, float* J_out) {
  if (!J_out || l_max < 0 || l_max > kMaxL) return SO2_ERR_INVALID_ARGUMENT;
  float ident[wig_total(kMaxL)];
  wigner_generators(l_max, J_out, ident);
  return SO2_OK;
}

}  // extern "C"

namespace so2 {

size_t attention_nowait_workspace_bytes(const so2_attn_desc* desc) {
  if (check_desc(desc) != SO2_OK) return 0;
  Kind kind = pick_kind(desc, &kBase, false);
  if (kind == kNone) return 0;
  return attn_layout(desc, kind).total;
}

so2_status attention_fwd_nowait(const so2_attn_desc* desc, const float* pos, const float* box_host,
                                const int32_t* row_ptr, const int32_t* col, const void* x, const void* w_q,
                                const void* w_k, const void* w_rad, const void* w_so2, float* y, void* workspace,
                                size_t workspace_bytes, so2_stream_t stream) {
  return attention_fwd_impl(SO2_STAGE_PREPARE | SO2_STAGE_FUSED, desc, &kBase, pos, box_host, row_ptr, col, x, w_q,
                            w_k, w_rad, w_so2, nullptr, nullptr, y, workspace, workspace_bytes, stream, false);
}

}  // namespace so2
