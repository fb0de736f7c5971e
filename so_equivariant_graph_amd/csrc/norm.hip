// Equivariant merged RMS layer norm of the node features.
//
// "EquiformerV3: Scaling Efficient, Expressive, and General SE(3)-Equivariant
// Graph Attention Transformers", technical summary, section 2.B.1: a single
// root-mean-square statistic is shared by every degree l >= 0 of a node, so
// the relative weight of the degrees survives the normalisation.  Reading:
//   y[(l, m), c] = gamma[l][c] x[(l, m), c] / sqrt(mean_{l, m, c} x^2 + eps)
// (gain per degree and channel, the same for the 2l + 1 components of a
// degree, so the map commutes with rotations; no centring, no bias).
//
// One wave per node, 4 nodes per block.  The node's (L+1)^2 C values are
// read once with 16-byte loads and kept in registers (up to 16 vectors per
// lane: 8192 bf16 or 4096 fp32 values per node) while their squares are
// summed in fp32 and reduced across the wave; then gamma x / rms is written,
// rounded to bf16 when the input is bf16.  Larger nodes read x twice.  Every
// element is read before the same lane writes it, so y may alias x.
#include "norm.h"

#include "launch.h"

namespace so2 {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4n;
typedef __attribute__((ext_vector_type(4))) float f32x4n;

template <typename T>
struct NormVec;  // 16 bytes of T
template <>
struct NormVec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float (&v)[8]) { unpack(*(const u32x4n*)p, v); }
  __device__ static void unpack(const u32x4n w, float (&v)[8]) {
    const unsigned int a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_float((uint16_t)(a[i] & 0xffffu));
      v[2 * i + 1] = bf16_to_float((uint16_t)(a[i] >> 16));
    }
  }
  __device__ static void store(uint16_t* p, const float (&v)[8]) {
    u32x4n w;
    unsigned int a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = (uint32_t)float_to_bf16(v[2 * i]) | ((uint32_t)float_to_bf16(v[2 * i + 1]) << 16);
    w.x = a[0];
    w.y = a[1];
    w.z = a[2];
    w.w = a[3];
    *(u32x4n*)p = w;
  }
};
template <>
struct NormVec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float (&v)[4]) { unpack(*(const u32x4n*)p, v); }
  __device__ static void unpack(const u32x4n u, float (&v)[4]) {
    const f32x4n w = __builtin_bit_cast(f32x4n, u);
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
  }
  __device__ static void store(float* p, const float (&v)[4]) { *(f32x4n*)p = f32x4n{v[0], v[1], v[2], v[3]}; }
};

// degree of component row comp = l^2 .. l^2 + 2l
__device__ inline int comp_degree(int comp) {
  int l = 0;
  while ((l + 1) * (l + 1) <= comp) ++l;
  return l;
}

// Register path: C % N == 0, 16-byte aligned x and y, at most 64 MV
// vectors per node (MV = 8 or 16).
constexpr int kMaxVec = 16;
template <typename T, int MV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MV <= 8 ? 4 : 2)))
merged_rms_norm_reg_kernel(const T* x, const float* __restrict__ gamma, T* y, int n_atoms, int nc, int C, float eps) {
  constexpr int N = NormVec<T>::N;
  const int lane = threadIdx.x & 63;
  const int node = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (node >= n_atoms) return;
  const int64_t ne = (int64_t)nc * C;
  const T* xn = x + (int64_t)node * ne;
  T* yn = y + (int64_t)node * ne;
  const int nv = (int)(ne / N);
  u32x4n raw[MV];  // the node's values as loaded (bf16 or fp32 bits)
#pragma unroll
  for (int k = 0; k < MV; ++k) {
    const int v = lane + 64 * k;
    if (v < nv) raw[k] = *(const u32x4n*)(xn + (int64_t)v * N);
  }
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < MV; ++k)
    if (lane + 64 * k < nv) {
      float a[N];
      NormVec<T>::unpack(raw[k], a);
#pragma unroll
      for (int i = 0; i < N; ++i) ss += a[i] * a[i];
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float inv = 1.0f / sqrtf(ss / (float)ne + eps);
#pragma unroll
  for (int k = 0; k < MV; ++k) {
    const int v = lane + 64 * k;
    if (v < nv) {
      const int e = v * N, comp = e / C, c0 = e % C;
      const float* g = gamma + (int64_t)comp_degree(comp) * C + c0;
      float a[N];
      NormVec<T>::unpack(raw[k], a);
#pragma unroll
      for (int i = 0; i < N; ++i) a[i] = a[i] * inv * g[i];
      NormVec<T>::store(yn + e, a);
    }
  }
}

// Vector path: C % N == 0 and 16-byte aligned x and y; reads x twice.
template <typename T>
__global__ void __launch_bounds__(256) merged_rms_norm_kernel(const T* x, const float* __restrict__ gamma, T* y,
                                                              int n_atoms, int nc, int C, float eps) {
  constexpr int N = NormVec<T>::N;
  const int lane = threadIdx.x & 63;
  const int node = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (node >= n_atoms) return;
  const int64_t ne = (int64_t)nc * C;
  const T* xn = x + (int64_t)node * ne;
  T* yn = y + (int64_t)node * ne;
  const int nv = (int)(ne / N);
  float ss = 0.0f;
  for (int v = lane; v < nv; v += 64) {
    float a[N];
    NormVec<T>::load(xn + (int64_t)v * N, a);
#pragma unroll
    for (int i = 0; i < N; ++i) ss += a[i] * a[i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float inv = 1.0f / sqrtf(ss / (float)ne + eps);
  for (int v = lane; v < nv; v += 64) {
    const int e = v * N, comp = e / C, c0 = e % C;
    const float* g = gamma + (int64_t)comp_degree(comp) * C + c0;
    float a[N];
    NormVec<T>::load(xn + e, a);
#pragma unroll
    for (int i = 0; i < N; ++i) a[i] = a[i] * inv * g[i];
    NormVec<T>::store(yn + e, a);
  }
}

// Element path for any C and alignment.
template <typename T>
__global__ void __launch_bounds__(256) merged_rms_norm_any_kernel(const T* x, const float* __restrict__ gamma, T* y,
                                                                  int n_atoms, int nc, int C, float eps) {
  const int lane = threadIdx.x & 63;
  const int node = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (node >= n_atoms) return;
  const int64_t ne = (int64_t)nc * C;
  const T* xn = x + (int64_t)node * ne;
  T* yn = y + (int64_t)node * ne;
  float ss = 0.0f;
  for (int64_t e = lane; e < ne; e += 64) {
    const float a = load_as_float(xn, e);
    ss += a * a;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float inv = 1.0f / sqrtf(ss / (float)ne + eps);
  for (int64_t e = lane; e < ne; e += 64) {
    const int comp = (int)(e / C), c = (int)(e % C);
    const float v = load_as_float(xn, e) * inv * gamma[(int64_t)comp_degree(comp) * C + c];
    if constexpr (sizeof(T) == 2) yn[e] = float_to_bf16(v);
    else yn[e] = v;
  }
}

so2_status launch_merged_rms_norm(const void* x, const float* gamma, void* y, int n_atoms, int L, int C,
                                  float eps, int dtype, hipStream_t stream) {
  if (n_atoms == 0) return SO2_OK;
  const int nc = n_comp(L);
  const dim3 grid((unsigned)((n_atoms + 3) / 4)), block(256);
  const bool aligned = !(((uintptr_t)x & 15) || ((uintptr_t)y & 15));
  const int64_t ne = (int64_t)nc * C;
  if (dtype == SO2_BF16) {
    if (aligned && C % 8 == 0 && ne / 8 <= 64 * 8)
      hipLaunchKernelGGL((merged_rms_norm_reg_kernel<uint16_t, 8>), grid, block, 0, stream, (const uint16_t*)x, gamma,
                         (uint16_t*)y, n_atoms, nc, C, eps);
    else if (aligned && C % 8 == 0 && ne / 8 <= 64 * kMaxVec)
      hipLaunchKernelGGL((merged_rms_norm_reg_kernel<uint16_t, kMaxVec>), grid, block, 0, stream, (const uint16_t*)x,
                         gamma, (uint16_t*)y, n_atoms, nc, C, eps);
    else if (aligned && C % 8 == 0)
      hipLaunchKernelGGL(merged_rms_norm_kernel<uint16_t>, grid, block, 0, stream, (const uint16_t*)x, gamma,
                         (uint16_t*)y, n_atoms, nc, C, eps);
    else
      hipLaunchKernelGGL(merged_rms_norm_any_kernel<uint16_t>, grid, block, 0, stream, (const uint16_t*)x, gamma,
                         (uint16_t*)y, n_atoms, nc, C, eps);
  } else {
    if (aligned && C % 4 == 0 && ne / 4 <= 64 * 8)
      hipLaunchKernelGGL((merged_rms_norm_reg_kernel<float, 8>), grid, block, 0, stream, (const float*)x, gamma,
                         (float*)y, n_atoms, nc, C, eps);
    else if (aligned && C % 4 == 0 && ne / 4 <= 64 * kMaxVec)
      hipLaunchKernelGGL((merged_rms_norm_reg_kernel<float, kMaxVec>), grid, block, 0, stream, (const float*)x, gamma,
                         (float*)y, n_atoms, nc, C, eps);
    else if (aligned && C % 4 == 0)
      hipLaunchKernelGGL(merged_rms_norm_kernel<float>, grid, block, 0, stream, (const float*)x, gamma, (float*)y,
                         n_atoms, nc, C, eps);
    else
      hipLaunchKernelGGL(merged_rms_norm_any_kernel<float>, grid, block, 0, stream, (const float*)x, gamma,
                         (float*)y, n_atoms, nc, C, eps);
  }
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

}  // namespace so2
