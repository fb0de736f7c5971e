// Invariant query/key projections.
//
// "E2Former-V2: On-the-Fly Equivariant Attention with Linear Activation
// Memory", technical summary, section 2.2: query and key vectors are built
// from SO(3)-invariant scalar projections, so only the value path carries
// geometry.  The invariant scalars of a node are its l = 0 channels:
//   q_i[o] = sum_c x_i[0][c] W_q[c][o],   k_j[o] = sum_c x_j[0][c] W_k[c][o].
// q is needed for the targets only, k for every atom.  fp32 accumulation.
#include "common.h"
#include "launch.h"

namespace so2 {

template <typename T>
__global__ void qk_proj_kernel(const T* __restrict__ x, const T* __restrict__ wq,
                               const T* __restrict__ wk, float* __restrict__ q,
                               float* __restrict__ k, int n_atoms, int n_targets, int nc, int C) {
  int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_atoms * C) return;
  int atom = (int)(idx / C);
  int o = (int)(idx % C);
  const T* xa = x + (int64_t)atom * nc * C;  // l = 0 row
  float aq = 0.0f, ak = 0.0f;
  const bool want_q = atom < n_targets;
  for (int c = 0; c < C; ++c) {
    float xv = load_as_float(xa, c);
    ak += xv * load_as_float(wk, (int64_t)c * C + o);
    if (want_q) aq += xv * load_as_float(wq, (int64_t)c * C + o);
  }
  k[idx] = ak;
  if (want_q) q[idx] = aq;
}

so2_status launch_qk_proj(const AttnArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.n_atoms * a.C;
  const int tb = 256;
  const int64_t blocks = (total + tb - 1) / tb;
  const int nc = n_comp(a.L);
  if (a.dtype == SO2_BF16) {
    hipLaunchKernelGGL(qk_proj_kernel<uint16_t>, dim3((unsigned)blocks), dim3(tb), 0, stream,
                       (const uint16_t*)a.x, (const uint16_t*)a.w_q, (const uint16_t*)a.w_k, a.q,
                       a.k, a.n_atoms, a.n_targets, nc, a.C);
  } else {
    hipLaunchKernelGGL(qk_proj_kernel<float>, dim3((unsigned)blocks), dim3(tb), 0, stream,
                       (const float*)a.x, (const float*)a.w_q, (const float*)a.w_k, a.q, a.k,
                       a.n_atoms, a.n_targets, nc, a.C);
  }
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

}  // namespace so2
