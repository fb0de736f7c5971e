// Edge frame and Wigner-D blocks for real spherical harmonics, computed in
// fp32 on the device (and, for tests, on the host by the same code).
//
// "E2Former-V2: On-the-Fly Equivariant Attention with Linear Activation
// Memory", technical summary, section 2.1 (EAAS): every edge is processed
// in the frame whose z axis is the edge vector.  The frame here is
//
//   R = R_y(-theta) R_z(-phi) = [[ct cp, ct sp, -st], [-sp, cp, 0], [x, y, z]]
//
// for rhat = (x, y, z) = (st cp, st sp, ct); it maps rhat to +z.  At the
// poles (st = 0) cp = 1, sp = 0.  Any frame with the same z axis gives the
// same layer output, because the per-m maps commute with rotations about z.
//
// D^l(R) satisfies Y_l(R s) = D^l(R) Y_l(s) in the basis of
// include/so2attn.h (real harmonics, no Condon-Shortley phase, l = 1 is
// (y, z, x)).  D^0 = 1, D^1 is R written in (y, z, x) order, and D^l for
// l >= 2 follows from D^{l-1} and D^1 by the recursion of J. Ivanic and
// K. Ruedenberg, "Rotation Matrices for Real Spherical Harmonics. Direct
// Determination by Recursion", J. Phys. Chem. 100, 6342 (1996), with the
// corrections in J. Phys. Chem. A 102, 9099 (1998).
#pragma once

#include <math.h>

#include "common.h"

namespace so2 {

// Frame rotation (row-major 3x3) for a normalised direction.
__host__ __device__ inline void edge_frame(float x, float y, float z, float* R) {
  float st = sqrtf(x * x + y * y);
  float cp = 1.0f, sp = 0.0f;
  if (st > 0.0f) {
    cp = x / st;
    sp = y / st;
  }
  float ct = z;
  R[0] = ct * cp;
  R[1] = ct * sp;
  R[2] = -st;
  R[3] = -sp;
  R[4] = cp;
  R[5] = 0.0f;
  R[6] = x;
  R[7] = y;
  R[8] = z;
}

// D^1 in (y, z, x) order, i.e. D1[(a+1)*3 + (b+1)] for a, b in {-1, 0, 1}.
__host__ __device__ inline void wigner_l1(const float* R, float* D1) {
  // axis of m: -1 -> y (1), 0 -> z (2), 1 -> x (0)
  const int ax[3] = {1, 2, 0};
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b) D1[a * 3 + b] = R[ax[a] * 3 + ax[b]];
}

// One entry D^l[m][mp] (l >= 2) from D^1 (3x3, m-ordered) and D^{l-1}
// ((2l-1)^2 row-major, m-ordered).
__host__ __device__ __attribute__((always_inline)) inline float wigner_entry(int l, int m, int mp,
                                                                           const float* D1,
                                                                           const float* Dp) {
  const int lp = l - 1;
  const int np = 2 * lp + 1;
  auto r1 = [&](int i, int j) { return D1[(i + 1) * 3 + (j + 1)]; };
  auto rp = [&](int mu, int nu) { return Dp[(mu + lp) * np + (nu + lp)]; };
  auto P = [&](int i, int mu) -> float {
    if (mp > -l && mp < l) return r1(i, 0) * rp(mu, mp);
    if (mp == l) return r1(i, 1) * rp(mu, l - 1) - r1(i, -1) * rp(mu, -l + 1);
    return r1(i, 1) * rp(mu, -l + 1) + r1(i, -1) * rp(mu, l - 1);
  };
  const int am = m < 0 ? -m : m;
  const float den = (mp > -l && mp < l) ? (float)((l + mp) * (l - mp)) : (float)(2 * l * (2 * l - 1));
  const float inv = 1.0f / den;
  float val = 0.0f;
  // U term: u = sqrt((l+m)(l-m)/den), nonzero for |m| < l
  if (am < l) val += sqrtf((float)((l + m) * (l - m)) * inv) * P(0, m);
  // V term
  if (m == 0) {
    float v = -0.5f * sqrtf(2.0f * (float)((l - 1) * l) * inv);
    val += v * (P(1, 1) + P(-1, -1));
  } else {
    float v = 0.5f * sqrtf((float)((l + am - 1) * (l + am)) * inv);
    float V;
    if (m > 0) {
      V = (m == 1) ? 1.41421356237309515f * P(1, 0) : P(1, m - 1) - P(-1, -m + 1);
    } else {
      V = (m == -1) ? 1.41421356237309515f * P(-1, 0) : P(1, m + 1) + P(-1, -m - 1);
    }
    val += v * V;
  }
  // W term: w = -1/2 sqrt((l-|m|-1)(l-|m|)/den), nonzero for 0 < |m| < l-1
  if (m != 0 && am < l - 1) {
    float w = -0.5f * sqrtf((float)((l - am - 1) * (l - am)) * inv);
    float W = (m > 0) ? P(1, m + 1) + P(-1, -m - 1) : P(1, m - 1) - P(-1, -m + 1);
    val += w * W;
  }
  return val;
}

// All blocks D^0..D^L for one rotation, sequentially (host diagnostics and
// single-thread use).  D has wig_total(L) entries.
__host__ __device__ inline void wigner_blocks_serial(int L, const float* R, float* D) {
  D[0] = 1.0f;
  if (L < 1) return;
  float* D1 = D + wig_offset(1);
  wigner_l1(R, D1);
  for (int l = 2; l <= L; ++l) {
    const float* Dp = D + wig_offset(l - 1);
    float* Dl = D + wig_offset(l);
    const int n = 2 * l + 1;
    for (int a = 0; a < n; ++a)
      for (int b = 0; b < n; ++b) Dl[a * n + b] = wigner_entry(l, a - l, b - l, D1, Dp);
  }
}

// Generators of rotations in the real harmonic basis: J_a^l = d/dt
// D^l(exp(t [e_a]x)) at t = 0 for the axes a = x, y, z ([e_a]x v = e_a x v).
// The recursion is bilinear in (D^1, D^{l-1}) and D = I at t = 0, so
//   J^1 = (D^1 of [e_a]x),  J^l = f(J^1, I) + f(I, J^{l-1})
// with f the recursion step (wigner_entry).  J[a * wig_total(L) + ...]
// holds blocks 0..L like wigner_blocks_serial; each block is antisymmetric.
// ident must hold wig_total(L) floats of scratch.
__host__ __device__ inline void wigner_generators(int L, float* J, float* ident) {
  const int tot = wig_total(L);
  for (int q = 0; q < tot; ++q) ident[q] = 0.0f;
  for (int l = 0; l <= L; ++l)
    for (int a = 0; a < 2 * l + 1; ++a) ident[wig_offset(l) + a * (2 * l + 1) + a] = 1.0f;
  for (int ax = 0; ax < 3; ++ax) {
    float* Ja = J + ax * tot;
    Ja[0] = 0.0f;
    if (L < 1) continue;
    float E[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    if (ax == 0) {
      E[5] = -1.0f;
      E[7] = 1.0f;
    } else if (ax == 1) {
      E[2] = 1.0f;
      E[6] = -1.0f;
    } else {
      E[1] = -1.0f;
      E[3] = 1.0f;
    }
    float* J1 = Ja + wig_offset(1);
    wigner_l1(E, J1);
    const float* I1 = ident + wig_offset(1);
    for (int l = 2; l <= L; ++l) {
      const int n = 2 * l + 1;
      const float* Jp = Ja + wig_offset(l - 1);
      const float* Ip = ident + wig_offset(l - 1);
      float* Jl = Ja + wig_offset(l);
      for (int m = 0; m < n; ++m)
        for (int mp = 0; mp < n; ++mp)
          Jl[m * n + mp] = wigner_entry(l, m - l, mp - l, J1, Ip) + wigner_entry(l, m - l, mp - l, I1, Jp);
    }
  }
}

// D^l (l >= 2) from D^1 and D^{l-1}, all in registers: with l a template
// parameter every index, coefficient and branch of wigner_entry folds to a
// constant, leaving a few multiply-adds per entry.
template <int l>
__device__ __attribute__((always_inline)) inline void wigner_step(const float (&D1)[9],
                                                                  const float (&Dp)[(2 * l - 1) * (2 * l - 1)],
                                                                  float (&Dl)[(2 * l + 1) * (2 * l + 1)]) {
  constexpr int n = 2 * l + 1;
#pragma unroll
  for (int a = 0; a < n; ++a)
#pragma unroll
    for (int b = 0; b < n; ++b) Dl[a * n + b] = wigner_entry(l, a - l, b - l, D1, Dp);
}

// All blocks D^0..D^L of one rotation written to out[wig_total(L)], by one
// thread, in registers.
template <int L>
__device__ inline void wigner_blocks_unrolled(const float* R, float* out) {
  float D1[9];
  wigner_l1(R, D1);
  out[0] = 1.0f;
  if constexpr (L >= 1) {
#pragma unroll
    for (int q = 0; q < 9; ++q) out[wig_offset(1) + q] = D1[q];
  }
  if constexpr (L >= 2) {
    float D2[25];
    wigner_step<2>(D1, D1, D2);
#pragma unroll
    for (int q = 0; q < 25; ++q) out[wig_offset(2) + q] = D2[q];
    if constexpr (L >= 3) {
      float D3[49];
      wigner_step<3>(D1, D2, D3);
#pragma unroll
      for (int q = 0; q < 49; ++q) out[wig_offset(3) + q] = D3[q];
      if constexpr (L >= 4) {
        float D4[81];
        wigner_step<4>(D1, D3, D4);
#pragma unroll
        for (int q = 0; q < 81; ++q) out[wig_offset(4) + q] = D4[q];
        if constexpr (L >= 5) {
          float D5[121];
          wigner_step<5>(D1, D4, D5);
#pragma unroll
          for (int q = 0; q < 121; ++q) out[wig_offset(5) + q] = D5[q];
          if constexpr (L >= 6) {
            float D6[169];
            wigner_step<6>(D1, D5, D6);
#pragma unroll
            for (int q = 0; q < 169; ++q) out[wig_offset(6) + q] = D6[q];
          }
        }
      }
    }
  }
}

}  // namespace so2
