// Internal interface between the C-ABI entry points (abi.hip) and the
// translation units that own the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace so2 {

// Records the HIP error text for so2_last_device_error() and returns
// SO2_ERR_DEVICE.
so2_status device_error(hipError_t err);

#define SO2_CHECK(expr)                                      \
  do {                                                       \
    hipError_t so2_err_ = (expr);                            \
    if (so2_err_ != hipSuccess) return device_error(so2_err_); \
  } while (0)

#define SO2_CHECK_LAUNCH() SO2_CHECK(hipGetLastError())

// ---- neighbours (neighbors.hip)
size_t neighbors_workspace_bytes(int32_t n_atoms);
so2_status neighbors_build(const float* pos, int32_t n, const int32_t* mol_id,
                           const float* box_host, float cutoff, int32_t* row_ptr, int32_t* col,
                           int64_t capacity, int64_t* n_edges_host, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

// ---- attention
struct AttnArgs {
  const float* pos;
  const int32_t* row_ptr;
  const int32_t* col;
  const void* x;
  const void* w_q;
  const void* w_k;
  const void* w_rad;
  const void* w_so2;
  float* y;
  float* q;  // workspace [n_targets][C]
  float* k;  // workspace [n_atoms][C]
  void* scratch;  // kernel-specific workspace area
  size_t scratch_bytes;
  int32_t n_atoms, n_targets, L, C, H, K, p;
  float cutoff;
  uint32_t flags;
  int32_t dtype;
  int32_t periodic;
  float box[3];
  // variants (the base layer: m_max = L, n_focus = 1, no logit bias)
  int32_t m_max, n_focus;
  const void* w_logit;  // [K][H] or null
  const void* w_focus;  // [C] when n_focus > 1
};

// The base forward with a kernel that never waits on the stream (abi.hip):
// the MFMA kernel or the fp32 VALU kernel, for the no-allocation entry
// point, whose callers may be under stream capture.
size_t attention_nowait_workspace_bytes(const so2_attn_desc* desc);
so2_status attention_fwd_nowait(const so2_attn_desc* desc, const float* pos, const float* box_host,
                                const int32_t* row_ptr, const int32_t* col, const void* x, const void* w_q,
                                const void* w_k, const void* w_rad, const void* w_so2, float* y, void* workspace,
                                size_t workspace_bytes, so2_stream_t stream);

// q/k projection of the l = 0 slice (attention_prep.hip).
so2_status launch_qk_proj(const AttnArgs& a, hipStream_t stream);

// General kernel, fp32 arithmetic, any L <= 6, C <= 256 (attention_valu.hip).
bool valu_supported(int L, int C, int H);
size_t valu_scratch_bytes(int L, int C);
so2_status launch_attention_valu(const AttnArgs& a, hipStream_t stream);

// bf16 MFMA kernel (attention_mfma.hip): C = 128, 1 <= L <= 6, H <= 16, K <= 32
// (mfma_shape), up to the atom count its 32-bit buffer addressing covers
// (mfma_fits).  x, w_rad and w_so2 must be 16-byte aligned.
bool mfma_shape(int L, int C, int H, int K);
// focus streams the MFMA kernel takes (n_focus = 1: always)
bool mfma_focus(int L, int H, int m_max, int n_focus);
bool mfma_fits(int L, int n_atoms);
bool mfma_aligned(const AttnArgs& a);
size_t mfma_scratch_bytes(int n_atoms, int n_targets, int L, int H, int K);
// prologue (x repacked as component pairs, w_rad in fp32, w_so2 in fragment
// order), softmax statistics and the run schedule, all on `stream`; then the
// fused kernel alone
so2_status launch_attention_mfma_prep(const AttnArgs& a, hipStream_t stream);
so2_status launch_attention_mfma(const AttnArgs& a, hipStream_t stream);

// Backward (attention_batch.hip), fp32 arithmetic: any L <= 6, C <= 256,
// H <= 256.  Workspace beyond q, k: dq, dk, the softmax statistics and head
// sums per (target, head), the per-m maps in fp32 and their gradients, and
// the per-edge tensors of one batch of edges (batch_edges(n_targets)).
// dw_* may be null (not computed).  Reads the targets' edge range back to
// the host once (one stream synchronisation) to plan the batches.
bool bwd_supported(int L, int C, int H, int K);
size_t bwd_scratch_bytes(int n_atoms, int n_targets, int L, int C, int H, int K);
// fp32 forward on the same edge batches (attention_batch.hip): per-edge
// rotation kernels, the per-m maps as fp32 GEMMs on the matrix cores, a
// deterministic per-target sum; every variant (m_max, focus streams, logit
// bias).  Reads the targets' edge range back once (one stream wait).
bool batch_fwd_supported(int L, int C, int H, int K, int m_max, int n_focus);
size_t batch_fwd_scratch_bytes(int n_targets, int L, int C, int H, int m_max, int n_focus);
so2_status launch_attention_batch_fwd(const AttnArgs& a, hipStream_t stream);
so2_status launch_attention_bwd(const AttnArgs& a, const float* dy, float* dx, float* dpos, float* dw_q, float* dw_k,
                                float* dw_rad, float* dw_so2, hipStream_t stream);

}  // namespace so2
