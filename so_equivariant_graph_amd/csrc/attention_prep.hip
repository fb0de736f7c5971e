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

// Tiled version for C = 128: a block of 256 threads computes 32 atoms x 128
// outputs of q and k.  The atoms' l = 0 rows are staged in LDS in fp32;
// thread t owns output column t % 128 for the 16 atoms of half t / 128 and
// streams the weight rows from global memory (coalesced across the column
// index), four input channels at a time.
template <typename T>
__global__ void __launch_bounds__(256) qk_proj128_kernel(const T* __restrict__ x, const T* __restrict__ wq,
                                                         const T* __restrict__ wk, float* __restrict__ q,
                                                         float* __restrict__ k, int n_atoms, int n_targets,
                                                         int nc) {
  constexpr int C = 128, AB = 32, APT = 16;
  __shared__ __attribute__((aligned(16))) float xs[AB][C];
  const int t = threadIdx.x;
  const int a0 = blockIdx.x * AB;
  for (int i = t; i < AB * C; i += 256) {
    const int a = a0 + i / C;
    xs[i / C][i % C] = a < n_atoms ? load_as_float(x + (int64_t)a * nc * C, i % C) : 0.0f;
  }
  __syncthreads();
  const int o = t % C, g = t / C;
  const bool any_q = a0 + g * APT < n_targets;
  float aq[APT], ak[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) aq[i] = ak[i] = 0.0f;
  for (int c = 0; c < C; c += 4) {
    float wk4[4], wq4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wk4[j] = load_as_float(wk, (int64_t)(c + j) * C + o);
      wq4[j] = any_q ? load_as_float(wq, (int64_t)(c + j) * C + o) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const float4 xv = *(const float4*)&xs[g * APT + i][c];
      ak[i] += xv.x * wk4[0] + xv.y * wk4[1] + xv.z * wk4[2] + xv.w * wk4[3];
      aq[i] += xv.x * wq4[0] + xv.y * wq4[1] + xv.z * wq4[2] + xv.w * wq4[3];
    }
  }
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int a = a0 + g * APT + i;
    if (a < n_atoms) k[(int64_t)a * C + o] = ak[i];
    if (a < n_targets) q[(int64_t)a * C + o] = aq[i];
  }
}

so2_status launch_qk_proj(const AttnArgs& a, hipStream_t stream) {
  const int nc = n_comp(a.L);
  if (a.C == 128) {
    const int blocks = (a.n_atoms + 31) / 32;
    if (a.dtype == SO2_BF16)
      hipLaunchKernelGGL(qk_proj128_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const uint16_t*)a.x, (const uint16_t*)a.w_q, (const uint16_t*)a.w_k, a.q, a.k,
                         a.n_atoms, a.n_targets, nc);
    else
      hipLaunchKernelGGL(qk_proj128_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const float*)a.x, (const float*)a.w_q, (const float*)a.w_k, a.q, a.k, a.n_atoms,
                         a.n_targets, nc);
    SO2_CHECK_LAUNCH();
    return SO2_OK;
  }
  const int64_t total = (int64_t)a.n_atoms * a.C;
  const int tb = 256;
  const int64_t blocks = (total + tb - 1) / tb;
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
