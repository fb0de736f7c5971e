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
// Transformers", technical summary, section 2.B.3).  u(1) = u'(1) = u''(1) =
// 0, so u = (1 - s)^3 Q(s) with Q(s) = sum_{k<p} (k+1)(k+2)/2 s^k (the degree
// p-1 truncation of 1/(1-s)^3), a sum of positive terms: evaluated in that
// form from t = 1 - s it keeps its relative precision up to the cutoff,
// where the expanded sum cancels.  Arguments: s and t = 1 - s (t computed in
// fp64 by edge_geometry, since 1 - s formed in fp32 from an fp32 length loses
// the digits that decide u near the cutoff).
__host__ __device__ inline float envelope_u(float s, float t, int p) {
  if (!(t > 0.0f)) return 0.0f;
  float q = 0.0f;
  for (int k = p - 1; k >= 0; --k) q = q * s + 0.5f * (float)((k + 1) * (k + 2));
  return t * t * t * q;
}

// du/ds of envelope_u: -3 t^2 Q(s) + t^3 Q'(s), Q'(s) = sum_{1<=k<p} k (k+1)(k+2)/2 s^(k-1); 0 outside.
__host__ __device__ inline float envelope_du(float s, float t, int p) {
  if (!(t > 0.0f)) return 0.0f;
  float q = 0.0f, dq = 0.0f;
  for (int k = p - 1; k >= 0; --k) {
    const float ck = 0.5f * (float)((k + 1) * (k + 2));
    dq = dq * s + q;  // Horner for the derivative alongside the value
    q = q * s + ck;
  }
  return t * t * (t * dq - 3.0f * q);
}

// Geometry of edge (i -> j) from fp32 positions, in fp64: r = p_j - p_i
// (exact in fp64), with a box the minimum image r - b rint(r / b) (the
// operation sequence of the neighbour test, no contraction), |r| and
// t = 1 - |r| / rc.  r and |r| are returned in fp32.
struct EdgeGeo {
  float r[3];
  float rho;
  float s;  // |r| / rc
  float t;  // 1 - |r| / rc, from the fp64 length
};

__host__ __device__ inline EdgeGeo edge_geometry(const float* pos, int i, int j, int periodic, const float* box,
                                                 float cutoff) {
#pragma clang fp contract(off)
  EdgeGeo g;
  double r2 = 0.0;
  for (int d = 0; d < 3; ++d) {
    double v = (double)pos[3 * (int64_t)j + d] - (double)pos[3 * (int64_t)i + d];
    if (periodic) {
      const double b = (double)box[d];
      v = v - b * rint(v / b);
    }
    r2 = r2 + v * v;
    g.r[d] = (float)v;
  }
  const double rho = sqrt(r2);
  const double rc = (double)cutoff;
  g.rho = (float)rho;
  g.s = (float)(rho / rc);
  g.t = (float)((rc - rho) / rc);
  return g;
}

}  // namespace so2
