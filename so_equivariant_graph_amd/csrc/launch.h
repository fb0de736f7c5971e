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
  int64_t n_edges;  // edges of the target rows (from the descriptor)
  float cutoff;
  uint32_t flags;
  int32_t dtype;
  int32_t periodic;
  float box[3];
};

// q/k projection of the l = 0 slice (attention_prep.hip).
so2_status launch_qk_proj(const AttnArgs& a, hipStream_t stream);

// General kernel, fp32 arithmetic, any L <= 6, C <= 256 (attention_valu.hip).
bool valu_supported(int L, int C, int H);
size_t valu_scratch_bytes(int L, int C);
so2_status launch_attention_valu(const AttnArgs& a, hipStream_t stream);

// bf16 MFMA kernel (attention_mfma.hip): C = 128, 1 <= L <= 6, H <= 16, K <= 32.
// x, w_rad and w_so2 must be 16-byte aligned.
bool mfma_supported(int L, int C, int H, int K, int n_atoms);
bool mfma_aligned(const AttnArgs& a);
size_t mfma_scratch_bytes(int n_atoms, int n_targets, int L, int H, int K);
// prologue (x repacked as component pairs, w_rad in fp32, w_so2 in fragment
// order), softmax statistics and the run schedule; then the fused kernel
// alone
so2_status launch_attention_mfma_prep(const AttnArgs& a, hipStream_t stream);
so2_status launch_attention_mfma(const AttnArgs& a, hipStream_t stream);

}  // namespace so2
