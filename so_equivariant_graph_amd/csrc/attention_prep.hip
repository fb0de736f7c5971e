// Invariant query/key projections.
//
// "E2Former-V2: On-the-Fly Equivariant Attention with Linear Activation
// Memory", technical summary, section 2.2: query and key vectors are built
// from SO(3)-invariant scalar projections, so only the value path carries
// geometry.  The invariant scalars of a node are its l = 0 channels:
//   q_i[o] = sum_c x_i[0][c] W_q[c][o],   k_j[o] = sum_c x_j[0][c] W_k[c][o].
// q is needed for the targets only, k for every atom.  fp32 accumulation.
#include <stdint.h>

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

// bf16, C = 128, on the matrix cores (v_mfma_f32_16x16x32_bf16; the bf16
// products are exact in fp32, so the result differs from the fp32 loop only
// in summation order).  A block of 4 waves takes 64 atoms; wave w computes
// atoms 16 w .. 16 w + 15 against all 256 outputs (q then k): 16 column
// tiles x 4 K steps.  A fragments (8 consecutive input channels of one
// atom's l = 0 row) load straight from x; the B fragments need 8
// consecutive input channels of one output column, so the block first
// stages W_q and W_k transposed in LDS, wt[m][o][c], with the 16-byte groups
// of each row XOR-swizzled by o % 16 so that the 16 lanes of a fragment
// read touch 16 different bank groups.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__device__ inline int wt_off(int o, int c) {  // element offset of wt[o][c] within one matrix
  return o * 128 + 8 * ((c >> 3) ^ (o & 15)) + (c & 7);
}

__global__ void __launch_bounds__(256) qk_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ wk, float* __restrict__ q,
                                                      float* __restrict__ k, int n_atoms, int n_targets, int nc) {
  constexpr int C = 128;
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][C * C];
  const int t = threadIdx.x;
  const int a0 = blockIdx.x * 64;
  const bool want_q = a0 < n_targets;
  // transposed staging: thread tile = input rows c, c + 1 x outputs o .. o + 7
  for (int tile = t; tile < 2 * (C / 2) * (C / 8); tile += 256) {
    const int m = tile / ((C / 2) * (C / 8));
    if (m == 0 && !want_q) continue;
    const int r = tile % ((C / 2) * (C / 8));
    const int c = 2 * (r / (C / 8)), o = 8 * (r % (C / 8));
    const uint16_t* w = m == 0 ? wq : wk;
    const u32x4_t lo = *(const u32x4_t*)(w + (int64_t)c * C + o);
    const u32x4_t hi = *(const u32x4_t*)(w + (int64_t)(c + 1) * C + o);
    const unsigned int l4[4] = {lo.x, lo.y, lo.z, lo.w}, h4[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned int vl = (l4[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      const unsigned int vh = (h4[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      *(unsigned int*)&wt[m][wt_off(o + i, c)] = vl | (vh << 16);
    }
  }
  __syncthreads();
  const int lane = t & 63, w = t >> 6;
  const int row0 = a0 + 16 * w;
  if (row0 >= n_atoms) return;
  const int ar = row0 + (lane & 15);  // atom of this lane's A rows
  const int g = lane >> 4;
  u32x4_t af[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    af[ks] = ar < n_atoms ? *(const u32x4_t*)(x + (int64_t)ar * nc * C + 32 * ks + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
  const bool wave_q = row0 < n_targets;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (m == 0 && !wave_q) continue;
    float* out = m == 0 ? q : k;
    const int lim = m == 0 ? n_targets : n_atoms;
#pragma unroll
    for (int ot = 0; ot < C / 16; ++ot) {
      const int o = 16 * ot + (lane & 15);
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t bf = *(const u32x4_t*)&wt[m][wt_off(o, 32 * ks + 8 * g)];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[ks]),
                                                      __builtin_bit_cast(bf16x8_t, bf), acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = row0 + 4 * g + i;
        if (a < lim) out[(int64_t)a * C + o] = acc[i];
      }
    }
  }
}

so2_status launch_qk_proj(const AttnArgs& a, hipStream_t stream) {
  const int nc = n_comp(a.L);
  const bool aligned = !(((uintptr_t)a.x & 15) || ((uintptr_t)a.w_q & 15) || ((uintptr_t)a.w_k & 15));
  if (a.C == 128 && a.dtype == SO2_BF16 && aligned) {
    hipLaunchKernelGGL(qk_mfma_kernel, dim3((unsigned)((a.n_atoms + 63) / 64)), dim3(256), 0, stream,
                       (const uint16_t*)a.x, (const uint16_t*)a.w_q, (const uint16_t*)a.w_k, a.q, a.k, a.n_atoms,
                       a.n_targets, nc);
    SO2_CHECK_LAUNCH();
    return SO2_OK;
  }
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
