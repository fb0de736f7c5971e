// Shared helpers for the HIP kernels and the C-ABI host code (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "so2attn.h"

namespace so2 {

constexpr int kMaxL = 6;

// Number of irreps components up to degree L: (L+1)^2.
__host__ __device__ constexpr int n_comp(int L) { return (L + 1) * (L + 1); }

// Offset of the Wigner-D block of degree l when the blocks D^0..D^L are
// stored back to back, each (2l+1)^2 row-major: sum_{k<l} (2k+1)^2.
__host__ __device__ constexpr int wig_offset(int l) { return l * (4 * l * l - 1) / 3; }

// Total Wigner-D entries for degrees 0..L.
__host__ __device__ constexpr int wig_total(int L) { return wig_offset(L + 1); }

// Offsets of the SO(2) weight blocks in the packed w_so2 layout.
// W0 first, then (W1_m, W2_m) for m = 1..L; block m has (L+1-m)C rows/cols.
__host__ __device__ inline int64_t so2_w1_offset(int L, int C, int m) {
  int64_t k0 = (int64_t)(L + 1) * C;
  int64_t off = k0 * k0;
  for (int mu = 1; mu < m; ++mu) {
    int64_t km = (int64_t)(L + 1 - mu) * C;
    off += 2 * km * km;
  }
  return off;
}

// bf16 <-> fp32.  bf16 is the top half of an fp32; widening is exact.
__host__ __device__ inline float bf16_to_float(uint16_t b) {
  union {
    uint32_t u;
    float f;
  } v;
  v.u = ((uint32_t)b) << 16;
  return v.f;
}

// Round to nearest even (finite inputs).
__host__ __device__ inline uint16_t float_to_bf16(float f) {
  union {
    uint32_t u;
    float f;
  } v;
  v.f = f;
  uint32_t r = v.u + 0x7FFFu + ((v.u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

template <typename T>
__device__ inline float load_as_float(const T* p, int64_t i);

template <>
__device__ inline float load_as_float<float>(const float* p, int64_t i) {
  return p[i];
}

template <>
__device__ inline float load_as_float<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_float(p[i]);
}

// Envelope u(s) = 1 - (p+1)(p+2)/2 s^p + p(p+2) s^(p+1) - p(p+1)/2 s^(p+2)
// for s < 1, else 0 (smooth radius cutoff inside attention: "EquiformerV3:
// Scaling Efficient, Expressive, and General SE(3)-Equivariant Graph Attention
// Transformers",
// technical summary, section 2.B.3).
__device__ inline float envelope_u(float s, int p) {
  if (!(s < 1.0f)) return 0.0f;
  float sp = 1.0f;
  for (int k = 0; k < p; ++k) sp *= s;
  const float a = 0.5f * (float)((p + 1) * (p + 2));
  const float b = (float)(p * (p + 2));
  const float c = 0.5f * (float)(p * (p + 1));
  return 1.0f + sp * (-a + s * (b - c * s));
}

}  // namespace so2
