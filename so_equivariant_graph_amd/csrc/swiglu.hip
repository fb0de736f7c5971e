// SwiGLU-S2 activation of node features.
//
// "EquiformerV3: Scaling Efficient, Expressive, and General SE(3)-Equivariant
// Graph Attention Transformers", technical summary, section 2.C: the features
// go to a grid on the sphere, the nonlinear gate acts on the scalar channels
// only and the grid features are multiplied bilinearly.  Reading, for node
// features x[(l, m), c] with per-degree channel maps A_l, B_l, O_l and a
// scalar map G (C x C, [in][out]):
//   u = x A_l, v = x B_l (per degree),  g = x[(0, 0)] G
//   h[(l, m)] = sum_p w_p Y_lm(r_p) u(r_p) v(r_p)   for l <= L
//   y[(l, m)] = (SiLU(g) h[(l, m)]) O_l
// on the product grid of n_t = ceil((3L + 1) / 2) Gauss-Legendre nodes in
// cos(theta) times n_f = 3L + 1 equally spaced phi.  u v has degree <= 2L and
// its projection onto degree <= L integrates degree <= 3L polynomials, which
// this grid does exactly, so the map is equivariant.
//
// Kernels:
// * the per-degree maps: bf16 with C = 128 on the matrix cores
//   (lin_mfma_kernel: a block stages one degree's C x C matrices transposed
//   in LDS and runs 64 nodes through them; u and v are kept in bf16, the
//   gate and y in fp32), every other shape on a plain loop in fp32
//   (lin_kernel);
// * bf16 with C = 128 and L <= 4, when the whole call is asked for: one
//   fused kernel (swiglu_fused_kernel, below) for maps, grid step and output
//   map, bitwise the same results as the three steps;
// * the grid step (s2_kernel): one wave per node, one lane per channel.  The
//   grid factorises, Y_lm(theta_i, phi_j) = Pn_lm(theta_i) T_m(phi_j) with
//   T_0 = 1, T_m = cos(m phi), T_-m = sin(m phi), so u on ring i is
//   sum_m F_m T_m(phi_j) with F_m = sum_l Pn_lm(theta_i) u_lm, and the
//   projection runs the same two sums in reverse.  Both factors have a mirror
//   symmetry (rings at +-cos(theta), meridians at +-phi) that halves each
//   sum again.  The tables Pn and T are built on the host and passed as
//   kernel arguments (read with scalar loads).
#include "swiglu.h"

#include <math.h>

#include <algorithm>

#include "launch.h"

namespace so2 {
namespace {

constexpr int kMaxNt = (3 * kMaxL + 2) / 2;  // Gauss-Legendre nodes at L = 6
constexpr double kPi = 3.14159265358979323846;

// The product grid: cos(theta_i) and the weight of every point of ring i,
// w_GL(i) 2 pi / n_f.
struct GridArgs {
  double ct[kMaxNt];
  double wt[kMaxNt];
};

// Gauss-Legendre nodes and weights of order n: the roots of P_n by Newton's
// method from cos(pi (i + 3/4) / (n + 1/2)), weights 2 / ((1 - x^2) P_n'(x)^2).
void gauss_legendre(int n, double* x_out, double* w_out) {
  for (int i = 0; i < n; ++i) {
    double x = cos(kPi * (i + 0.75) / (n + 0.5));
    double dp = 1.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = x;  // P_0, P_1
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2 * k - 1) * x * p1 - (k - 1) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (x * p1 - p0) / (x * x - 1.0);
      const double dx = p1 / dp;
      x -= dx;
      if (fabs(dx) < 1e-16) break;
    }
    double p0 = 1.0, p1 = x;
    for (int k = 2; k <= n; ++k) {
      const double p2 = ((2 * k - 1) * x * p1 - (k - 1) * p0) / k;
      p0 = p1;
      p1 = p2;
    }
    dp = n * (x * p1 - p0) / (x * x - 1.0);
    x_out[i] = x;
    w_out[i] = 2.0 / ((1.0 - x * x) * dp * dp);
  }
}

GridArgs make_grid(int L) {
  GridArgs g{};
  const int nt = (3 * L + 2) / 2, nf = 3 * L + 1;
  if (nt == 1) {
    g.ct[0] = 0.0;
    g.wt[0] = 2.0 * 2.0 * kPi / nf;
    return g;
  }
  double x[kMaxNt], w[kMaxNt];
  gauss_legendre(nt, x, w);
  for (int i = 0; i < nt; ++i) {
    g.ct[i] = x[i];
    g.wt[i] = w[i] * 2.0 * kPi / nf;
  }
  return g;
}

// Pn_k(x) for component k = (l, m): the theta factor of the real harmonic,
// sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) P_l^|m|(x), times sqrt(2) for m != 0;
// P_l^m without the (-1)^m phase, by the recurrences P_m^m = (2m-1)!! s^m,
// P_{m+1}^m = (2m+1) x P_m^m, (l-m) P_l^m = (2l-1) x P_{l-1}^m - (l+m-1) P_{l-2}^m.
__host__ __device__ double theta_factor(int k, double x) {
  int l = 0;
  while ((l + 1) * (l + 1) <= k) ++l;
  const int m = k - l * l - l, am = m < 0 ? -m : m;
  const double st = sqrt(fmax(0.0, 1.0 - x * x));
  double pmm = 1.0;
  for (int i = 1; i <= am; ++i) pmm *= (2 * i - 1) * st;
  double p = pmm;
  if (l > am) {
    double a = pmm, b = x * (2 * am + 1) * pmm;
    for (int ll = am + 2; ll <= l; ++ll) {
      const double c = ((2 * ll - 1) * x * b - (ll + am - 1) * a) / (ll - am);
      a = b;
      b = c;
    }
    p = b;
  }
  double ratio = 1.0;
  for (int i = l - am + 1; i <= l + am; ++i) ratio /= i;
  const double nrm = sqrt((2 * l + 1) / (4.0 * kPi) * ratio);
  return (m == 0 ? 1.0 : sqrt(2.0)) * nrm * p;
}

template <typename T>
__device__ inline void store_value(T* p, float v);
template <>
__device__ inline void store_value<float>(float* p, float v) {
  *p = v;
}
template <>
__device__ inline void store_value<uint16_t>(uint16_t* p, float v) {
  *p = float_to_bf16(v);
}

// The grid's tables: pn[i][k] = Pn_k(cos theta_i), tf[j][L + m] = T_m(phi_j)
// (zero past 2L + 1), wq[i] = the weight of every point of ring i.  Built on
// the host and passed by value, so the kernels read them from the kernel
// argument segment with scalar loads (the same value for every lane) instead
// of LDS.
template <int L>
struct S2Tables {
  static constexpr int NC = (L + 1) * (L + 1), NM = 2 * L + 1, NT = (3 * L + 2) / 2, NF = 3 * L + 1;
  static constexpr int NMP = (NM + 3) & ~3;
  float pn[NT][NC];
  float tf[NF][NMP];
  float wq[NT];
};

template <int L>
S2Tables<L> make_tables() {
  typedef S2Tables<L> S;
  const GridArgs grid = make_grid(L);
  S2Tables<L> T{};
  for (int i = 0; i < S::NT; ++i)
    for (int k = 0; k < S::NC; ++k) T.pn[i][k] = (float)theta_factor(k, grid.ct[i]);
  for (int j = 0; j < S::NF; ++j)
    for (int q = 0; q < S::NMP; ++q) {
      const int mm = q - L;
      const double ph = 2.0 * kPi * j / S::NF;
      T.tf[j][q] = mm > L ? 0.0f : (float)(mm == 0 ? 1.0 : mm > 0 ? cos(mm * ph) : sin(-mm * ph));
    }
  for (int i = 0; i < S::NT; ++i) T.wq[i] = (float)grid.wt[i];
  return T;
}

// One ring: the product of u and v at its NF meridians, projected onto the
// T_m, added to g.  phi_0 = 0 (T_m = 1 for m >= 0, 0 for m < 0) stands
// alone; phi_j and phi_{NF-j} share the cosines and have opposite sines, so
// each pair costs one cosine sum and one sine sum per field; for even NF,
// phi = pi stands alone too.
template <int L>
__device__ __attribute__((always_inline)) inline void s2_ring_phi(const S2Tables<L>& T, const float (&fu)[2 * L + 1],
                                                                  const float (&fv)[2 * L + 1],
                                                                  float (&g)[2 * L + 1]) {
  constexpr int NM = 2 * L + 1, NF = 3 * L + 1;
  {
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int q = L; q < NM; ++q) {
      a += fu[q];
      b += fv[q];
    }
    const float hp = a * b;
#pragma unroll
    for (int q = L; q < NM; ++q) g[q] += hp;
  }
  for (int j = 1; 2 * j < NF; ++j) {
    float cu = fu[L], cv = fv[L], su = 0.0f, sv = 0.0f;
#pragma unroll
    for (int m = 1; m <= L; ++m) {
      const float c = T.tf[j][L + m], sn = T.tf[j][L - m];
      cu += c * fu[L + m];
      cv += c * fv[L + m];
      su += sn * fu[L - m];
      sv += sn * fv[L - m];
    }
    const float h1 = (cu + su) * (cv + sv), h2 = (cu - su) * (cv - sv);
    const float hs = h1 + h2, hd = h1 - h2;
    g[L] += hs;
#pragma unroll
    for (int m = 1; m <= L; ++m) {
      g[L + m] += T.tf[j][L + m] * hs;
      g[L - m] += T.tf[j][L - m] * hd;
    }
  }
  if constexpr (NF % 2 == 0) {
    constexpr int j = NF / 2;
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int q = L; q < NM; ++q) {
      a += T.tf[j][q] * fu[q];
      b += T.tf[j][q] * fv[q];
    }
    const float hp = a * b;
#pragma unroll
    for (int q = L; q < NM; ++q) g[q] += T.tf[j][q] * hp;
  }
}

// The grid step of one (node, channel): hh[(l, m)] = sum_p w_p Y_lm(r_p)
// u(r_p) v(r_p) from the harmonic coefficients uu and vv.  Ring pairs: rings
// i and NT - 1 - i have opposite cos(theta), and Pn_lm(-x) = (-1)^(l+m)
// Pn_lm(x), so one sum over the even l + m terms and one over the odd ones
// serve both (F = E + O on ring i, E - O on its mirror); the projection back
// takes ga + gb or ga - gb by parity.
// uu(k) and vv(k) give the coefficients; with kReload they are fetched
// again for every ring pair (the fused kernel reads them from LDS there
// rather than holding 2 (L + 1)^2 registers).
template <int L, bool kReload = false, class UF, class VF>
__device__ __attribute__((always_inline)) inline void s2_column(const S2Tables<L>& T, UF uu, VF vv,
                                                                float (&hh)[(L + 1) * (L + 1)]) {
  constexpr int NC = (L + 1) * (L + 1), NM = 2 * L + 1, NT = (3 * L + 2) / 2;
#pragma unroll
  for (int k = 0; k < NC; ++k) hh[k] = 0.0f;
  for (int i = 0; i < (NT + 1) / 2; ++i) {
    if constexpr (kReload) asm volatile("" ::: "memory");
    const bool pair = 2 * i + 1 != NT;
    float eu[NM], ou[NM], ev[NM], ov[NM];
#pragma unroll
    for (int q = 0; q < NM; ++q) eu[q] = ou[q] = ev[q] = ov[q] = 0.0f;
#pragma unroll
    for (int l = 0; l <= L; ++l)
#pragma unroll
      for (int m = -l; m <= l; ++m) {
        const float p = T.pn[i][l * l + l + m];
        if (((l + m) & 1) == 0) {
          eu[m + L] += p * uu(l * l + l + m);
          ev[m + L] += p * vv(l * l + l + m);
        } else {
          ou[m + L] += p * uu(l * l + l + m);
          ov[m + L] += p * vv(l * l + l + m);
        }
      }
    float fu[NM], fv[NM], ga[NM], gb[NM];
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      fu[q] = eu[q] + ou[q];
      fv[q] = ev[q] + ov[q];
      ga[q] = gb[q] = 0.0f;
    }
    s2_ring_phi<L>(T, fu, fv, ga);
    if (pair) {
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        fu[q] = eu[q] - ou[q];
        fv[q] = ev[q] - ov[q];
      }
      s2_ring_phi<L>(T, fu, fv, gb);
    }
    const float w = T.wq[i];
#pragma unroll
    for (int l = 0; l <= L; ++l)
#pragma unroll
      for (int m = -l; m <= l; ++m) {
        const float gq = ((l + m) & 1) == 0 ? ga[m + L] + gb[m + L] : ga[m + L] - gb[m + L];
        hh[l * l + l + m] += T.pn[i][l * l + l + m] * (w * gq);
      }
  }
}

// s[(l, m), c] = SiLU(g_c) sum_p w_p Y_lm(r_p) u(r_p)_c v(r_p)_c, one wave per
// node (grid-stride over nodes), lanes over channels.
constexpr int kS2Threads = 256;
template <int L, typename TU, typename TS>
__global__ void __launch_bounds__(kS2Threads) __attribute__((amdgpu_waves_per_eu(L <= 3 ? 3 : 1))) s2_kernel(const TU* __restrict__ u, const TU* __restrict__ v,
                                                        const float* __restrict__ gate, TS* __restrict__ s,
                                                        int n_atoms, int C, const S2Tables<L> T) {
  constexpr int NC = (L + 1) * (L + 1);

  const int lane = threadIdx.x & 63;
  const int n_waves = gridDim.x * (kS2Threads / 64);
  for (int node = blockIdx.x * (kS2Threads / 64) + (threadIdx.x >> 6); node < n_atoms; node += n_waves) {
    for (int c = lane; c < C; c += 64) {
      const int64_t base = (int64_t)node * NC * C + c;
      float uu[NC], vv[NC], hh[NC];
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        uu[k] = load_as_float(u, base + (int64_t)k * C);
        vv[k] = load_as_float(v, base + (int64_t)k * C);
      }
      const float z = gate[(int64_t)node * C + c];
      const float sg = z / (1.0f + expf(-z));
      s2_column<L>(T, [&](int k) { return uu[k]; }, [&](int k) { return vv[k]; }, hh);
#pragma unroll
      for (int k = 0; k < NC; ++k) store_value(s + base + (int64_t)k * C, sg * hh[k]);
    }
  }
}

// out[n][k][o] = sum_c in[n][k][c] W[l(k)][c][o] for components k < ncp, one
// thread per output; node strides in elements.
template <typename TI, typename TW>
__global__ void __launch_bounds__(256) lin_kernel(const TI* __restrict__ in, int64_t in_stride,
                                                  const TW* __restrict__ W, float* __restrict__ out,
                                                  int64_t out_stride, int n_atoms, int ncp, int C) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_atoms * ncp * C) return;
  const int o = (int)(idx % C);
  const int k = (int)((idx / C) % ncp);
  const int64_t node = idx / ((int64_t)C * ncp);
  int l = 0;
  while ((l + 1) * (l + 1) <= k) ++l;
  const TI* row = in + node * in_stride + (int64_t)k * C;
  const TW* w = W + (int64_t)l * C * C + o;
  float acc = 0.0f;
  for (int c = 0; c < C; ++c) acc += load_as_float(row, c) * load_as_float(w, (int64_t)c * C);
  out[node * out_stride + (int64_t)k * C + o] = acc;
}

// bf16, C = 128, on the matrix cores (v_mfma_f32_16x16x32_bf16): block
// (blockIdx.x, l) runs the components of degree l of 64 nodes through NM
// matrices W_m[l] (NM = 2: A and B in one pass over x).  The matrices are
// staged transposed in LDS, wt[m][o][c], with the 16-byte groups of a row
// XOR-swizzled by o % 16 so that the 16 lanes of a B-fragment read hit 16
// different bank groups; A fragments (8 consecutive channels of one row) load
// straight from memory.  Wave w takes nodes 16 w .. 16 w + 15.
typedef __attribute__((ext_vector_type(8))) __bf16 sw_bf16x8;
typedef __attribute__((ext_vector_type(4))) float sw_f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int sw_u32x4;

__device__ inline int sw_wt_off(int o, int c) { return o * 128 + 8 * ((c >> 3) ^ (o & 15)) + (c & 7); }

constexpr int kLinNodes = 64;
template <int NM, typename TO>
__global__ void __launch_bounds__(256) lin_mfma_kernel(const uint16_t* __restrict__ in, int64_t in_stride,
                                                       const uint16_t* __restrict__ w0,
                                                       const uint16_t* __restrict__ w1, TO* __restrict__ out0,
                                                       TO* __restrict__ out1, int64_t out_stride, int n_atoms) {
  constexpr int C = 128;
  __shared__ __attribute__((aligned(16))) uint16_t wt[NM][C * C];
  const int l = blockIdx.y;
  const int t = threadIdx.x;
  for (int tile = t; tile < NM * (C / 2) * (C / 8); tile += 256) {
    const int m = tile / ((C / 2) * (C / 8));
    const int r = tile % ((C / 2) * (C / 8));
    const int c = 2 * (r / (C / 8)), o = 8 * (r % (C / 8));
    const uint16_t* w = (m == 0 ? w0 : w1) + (int64_t)l * C * C;
    const sw_u32x4 lo = *(const sw_u32x4*)(w + (int64_t)c * C + o);
    const sw_u32x4 hi = *(const sw_u32x4*)(w + (int64_t)(c + 1) * C + o);
    const unsigned int l4[4] = {lo.x, lo.y, lo.z, lo.w}, h4[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned int vl = (l4[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      const unsigned int vh = (h4[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      *(unsigned int*)&wt[m][sw_wt_off(o + i, c)] = vl | (vh << 16);
    }
  }
  __syncthreads();
  const int lane = t & 63;
  const int row0 = blockIdx.x * kLinNodes + 16 * (t >> 6);
  if (row0 >= n_atoms) return;
  const int ar = row0 + (lane & 15);
  const int g = lane >> 4;
  // A fragments of component k + 1 load while component k runs
  auto load_a = [&](int k, sw_u32x4 (&af)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      af[ks] = ar < n_atoms ? *(const sw_u32x4*)(in + (int64_t)ar * in_stride + (int64_t)k * C + 32 * ks + 8 * g)
                            : sw_u32x4{0u, 0u, 0u, 0u};
  };
  const int k_end = (l + 1) * (l + 1);
  sw_u32x4 an[4];
  load_a(l * l, an);
  for (int k = l * l; k < k_end; ++k) {
    // NM = 2: a compiler-only barrier, so that the B fragments are re-read
    // from LDS for every component instead of being held in 256 registers
    // (one wave per SIMD): 720 -> 640 us at 100k nodes.  The single-matrix
    // maps were slower that way and keep their fragments in registers.
    if constexpr (NM == 2) asm volatile("" ::: "memory");
    sw_u32x4 af[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) af[ks] = an[ks];
    if (k + 1 < k_end) load_a(k + 1, an);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      TO* out = m == 0 ? out0 : out1;
#pragma unroll
      for (int ot = 0; ot < C / 16; ++ot) {
        const int o = 16 * ot + (lane & 15);
        sw_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const sw_u32x4 bf = *(const sw_u32x4*)&wt[m][sw_wt_off(o, 32 * ks + 8 * g)];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sw_bf16x8, af[ks]),
                                                        __builtin_bit_cast(sw_bf16x8, bf), acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = row0 + 4 * g + i;
          if (a < n_atoms) store_value(out + (int64_t)a * out_stride + (int64_t)k * C + o, acc[i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fused path
//
// bf16, C = 128, L <= 4: the whole activation of a group of 4 nodes in one
// workgroup of 4 waves, nothing but x read and y written in HBM.  A
// workgroup holds 79 KB of LDS (x, u and v in bf16, the gate) and at most
// 256 registers a lane, so two run on a compute unit, and one's matrix-core
// steps overlap the other's grid step.  Each workgroup strides over groups:
//   0. the group's x (26 KB) is in LDS: copied by LDS DMA during the
//      previous group's grid step (sw_x_dma);
//   1. u = x A_l, v = x B_l and the gate map g = x[(0,0)] G on the matrix
//      cores, u and v rounded to bf16 into LDS (as the three-kernel path
//      rounds them in memory), g in fp32;
//   2. the grid step of every (node, channel), one thread each, its result
//      s = SiLU(g) h rounded to bf16 in place of u;
//   3. y = s O_l on the matrix cores, fp32 to memory.
// Rows of the matrix-core tiles are (component m, node n) pairs of one
// degree, R = 4 m + n, so degree l fills ceil((2l + 1) / 4) tiles of 16
// rows; wave w owns the output column tiles w and w + 4 (16 channels each).
// The weights come in fragment order (sw_pack_kernel), one 16-byte load per
// lane and fragment, those of the next degree in flight during the current
// one.  The grid step reads its tables from the kernel arguments and its
// coefficients from LDS once per ring pair (holding them would take 50 more
// registers a lane at L = 4).
constexpr int kSwNodes = 4;
constexpr int kSwThreads = 256;
constexpr int kSwWaves = kSwThreads / 64;

// fragment-ordered weights: fragment ((q, ks, ct), lane) holds W[32 ks + 8
// (lane / 16) + j][16 ct + lane % 16], j = 0..7, of matrix q: A_l, B_l, O_l
// at q = 3 l, 3 l + 1, 3 l + 2, and G at q = 3 (L + 1).
__device__ inline int sw_frag(int q, int ks, int ct) { return (q * 4 + ks) * 8 + ct; }

__global__ void __launch_bounds__(256) sw_pack_kernel(const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb,
                                                      const uint16_t* __restrict__ wo,
                                                      const uint16_t* __restrict__ wg, sw_u32x4* __restrict__ wp,
                                                      int L) {
  constexpr int C = 128;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int nq = 3 * (L + 1) + 1;
  if (idx >= (int64_t)nq * 32 * 64) return;
  const int lane = (int)(idx % 64), f = (int)(idx / 64);
  const int ct = f % 8, ks = (f / 8) % 4, q = f / 32;
  const uint16_t* w = q == 3 * (L + 1) ? wg : (q % 3 == 0 ? wa : q % 3 == 1 ? wb : wo) + (int64_t)(q / 3) * C * C;
  const int k0 = 32 * ks + 8 * (lane >> 4), o = 16 * ct + (lane & 15);
  unsigned int v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    v[j] = (unsigned int)w[(int64_t)(k0 + 2 * j) * C + o] | ((unsigned int)w[(int64_t)(k0 + 2 * j + 1) * C + o] << 16);
  wp[idx] = sw_u32x4{v[0], v[1], v[2], v[3]};
}

// bf16 element (node n, component k, channel c) of a [4 NC][128] LDS array:
// row n NC + k, its 16-byte groups XOR-swizzled by 4 (k % 4) + n, so that
// the 16 rows of a fragment read (4 nodes at four consecutive components)
// fall in 16 different bank groups, while the rows of one (node, channel)
// take only four swizzles (four base addresses, fixed offsets)
template <int NC>
__device__ inline int sw_lds(int n, int k, int c) {
  return (n * NC + k) * 128 + 8 * ((c >> 3) ^ (4 * (k & 3) + n)) + (c & 7);
}

// The group's x into sx by LDS DMA (global_load_lds_dwordx4: lane i of a
// wave writes the 16 bytes at LDS base + 16 i, no registers): wave w copies
// the 1 KB blocks b = w, w + 4, ... of sx (four 256-byte rows each), lane i
// row 4 b + i / 16, LDS group i % 16, which holds the row's 16-byte group
// (i % 16) ^ swizzle.  Rows of nodes past the last one read the last node
// (their outputs are never written).  Completion is waited for with vmcnt.
template <int NC>
__device__ inline void sw_x_dma(const uint16_t* __restrict__ x, int n0, int n_atoms, uint16_t* sx) {
  constexpr int NBLK = kSwNodes * NC / 4;  // 1 KB blocks
  const int lane = threadIdx.x & 63;
  for (int b = threadIdx.x >> 6; b < NBLK; b += kSwWaves) {
    const int r = 4 * b + (lane >> 4), n = r / NC, k = r % NC;
    const int node = min(n0 + n, n_atoms - 1);
    const int j = (lane & 15) ^ (4 * (k & 3) + n);
    __builtin_amdgcn_global_load_lds((const void*)(x + ((int64_t)node * NC + k) * 128 + 8 * j),
                                     (void __attribute__((address_space(3)))*)(sx + (size_t)b * 512), 16, 0, 0);
  }
}

// The per-degree maps of a group on the matrix cores, one column tile: for
// every degree l and every tile of its rows R = 4 m + n, the A fragments
// (row R's node n and component l^2 + m, zero past 2l + 1) from the LDS
// array src, times the weight fragments of that degree, which ld(l, w)
// loads one degree ahead: with kUV, w[0], w[1] are A_l, B_l and, for l = 0,
// w[2] is G (the gate map), and acc[0], acc[1], acc[2] are the u, v and gate
// tiles; otherwise w[0] is O_l and acc[0] the y tile.  out(l, m, n, acc, i)
// takes lane row i (row 16 t + 4 (lane / 16) + i) of each tile, for rows of
// the degree.
template <int L, int NC, bool kUV, class LD, class OUT>
__device__ __attribute__((always_inline)) inline void sw_map_tiles(const uint16_t* src, int l16, int g4, LD ld,
                                                                   OUT out) {
  constexpr int NB = kSwNodes, NW = kUV ? 3 : 1;
  const sw_f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  sw_u32x4 w[L + 1][NW][4];
  ld(0, w[0]);
#pragma unroll
  for (int l = 0; l <= L; ++l) {
    if (l < L) ld(l + 1, w[l + 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < (NB * (2 * l + 1) + 15) / 16; ++t) {
      const int R = 16 * t + l16, m = R / NB, n = R % NB;
      const bool ok = m <= 2 * l;
      const int k = l * l + (ok ? m : 0);
      sw_f32x4 acc[3] = {zero4, zero4, zero4};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const sw_u32x4 a = ok ? *(const sw_u32x4*)&src[sw_lds<NC>(n, k, 32 * ks + 8 * g4)] : sw_u32x4{0u, 0u, 0u, 0u};
        const sw_bf16x8 af = __builtin_bit_cast(sw_bf16x8, a);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(sw_bf16x8, w[l][0][ks]), acc[0], 0, 0, 0);
        if constexpr (kUV) {
          acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(sw_bf16x8, w[l][1][ks]), acc[1], 0, 0, 0);
          if (l == 0)
            acc[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(sw_bf16x8, w[l][2][ks]), acc[2], 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int Ro = 16 * t + 4 * g4 + i, mo = Ro / NB, no = Ro % NB;
        if (mo <= 2 * l) out(l, mo, no, acc, i);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int L>
__global__ void __launch_bounds__(kSwThreads) __attribute__((amdgpu_waves_per_eu(2))) swiglu_fused_kernel(const uint16_t* __restrict__ x,
                                                                  const sw_u32x4* __restrict__ wp,
                                                                  float* __restrict__ y, int n_atoms,
                                                                  const S2Tables<L> T) {
  constexpr int C = 128, NB = kSwNodes, NC = (L + 1) * (L + 1);
  __shared__ __attribute__((aligned(16))) uint16_t sx[NB * NC * C];  // x
  __shared__ __attribute__((aligned(16))) uint16_t su[NB * NC * C];  // u, then s
  __shared__ __attribute__((aligned(16))) uint16_t sv[NB * NC * C];
  __shared__ float sg[NB][C];

  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, l16 = lane & 15;
  const sw_f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const int n_groups = (n_atoms + NB - 1) / NB;
  if ((int)blockIdx.x >= n_groups) return;
  sw_x_dma<NC>(x, blockIdx.x * NB, n_atoms, sx);
  for (int grp = blockIdx.x; grp < n_groups; grp += gridDim.x) {
    const int n0 = grp * NB;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's x DMA is done
    __syncthreads();  // the group's x is in LDS; the previous group is done with su, sv, sg

    // 1. u, v and the gate
#pragma unroll 1
    for (int ct = threadIdx.x >> 6; ct < 8; ct += kSwWaves) {
      const int col = 16 * ct + l16;
      sw_map_tiles<L, NC, true>(
          sx, l16, g4,
          [&](int l, sw_u32x4 (&w)[3][4]) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              w[0][ks] = wp[sw_frag(3 * l, ks, ct) * 64 + lane];
              w[1][ks] = wp[sw_frag(3 * l + 1, ks, ct) * 64 + lane];
              if (l == 0) w[2][ks] = wp[sw_frag(3 * (L + 1), ks, ct) * 64 + lane];
            }
          },
          [&](int l, int mo, int no, const sw_f32x4* acc, int i) {
            su[sw_lds<NC>(no, l * l + mo, col)] = float_to_bf16(acc[0][i]);
            sv[sw_lds<NC>(no, l * l + mo, col)] = float_to_bf16(acc[1][i]);
            if (l == 0) sg[no][col] = acc[2][i];
          });
    }
    __syncthreads();

    // 2. the grid step, one (node, channel) per thread and pass; the next
    // group's x loads into sx (read last in step 1) meanwhile
    const int nxt = grp + gridDim.x;
    if (nxt < n_groups) sw_x_dma<NC>(x, nxt * NB, n_atoms, sx);
#pragma unroll 1
    for (int e = threadIdx.x; e < NB * C; e += kSwThreads) {
      const int n = e / C, c = e % C;
      if (n0 + n >= n_atoms) continue;
      float hh[NC];
      const float z = sg[n][c];
      const float sgm = z / (1.0f + expf(-z));
      s2_column<L, true>(T, [&](int k) { return bf16_to_float(su[sw_lds<NC>(n, k, c)]); },
                         [&](int k) { return bf16_to_float(sv[sw_lds<NC>(n, k, c)]); }, hh);
#pragma unroll
      for (int k = 0; k < NC; ++k) su[sw_lds<NC>(n, k, c)] = float_to_bf16(sgm * hh[k]);
    }
    __syncthreads();

    // 3. y = s O_l
#pragma unroll 1
    for (int ct = threadIdx.x >> 6; ct < 8; ct += kSwWaves) {
      const int col = 16 * ct + l16;
      sw_map_tiles<L, NC, false>(
          su, l16, g4,
          [&](int l, sw_u32x4 (&w)[1][4]) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) w[0][ks] = wp[sw_frag(3 * l + 2, ks, ct) * 64 + lane];
          },
          [&](int l, int mo, int no, const sw_f32x4* acc, int i) {
            if (n0 + no < n_atoms) y[((int64_t)(n0 + no) * NC + l * l + mo) * C + col] = acc[0][i];
          });
    }
  }
}

template <int L>
void launch_fused(const uint16_t* x, const sw_u32x4* wp, float* y, int n, hipStream_t stream) {
  const int groups = (n + kSwNodes - 1) / kSwNodes;
  const int blocks = std::max(1, std::min(groups, 512));
  hipLaunchKernelGGL((swiglu_fused_kernel<L>), dim3(blocks), dim3(kSwThreads), 0, stream, x, wp, y, n, make_tables<L>());
}

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

struct SwLayout {
  size_t u, v, g, s, total;
};

// the fused path's fragment-ordered weights: 3 (L + 1) + 1 matrices of 32 KB
size_t sw_packed_bytes(int L) { return (size_t)(3 * (L + 1) + 1) * 32 * 64 * sizeof(sw_u32x4); }

bool sw_fused_shape(int L, int C, int dtype) { return dtype == SO2_BF16 && C == 128 && L <= 4; }

SwLayout sw_layout(int n, int L, int C, int dtype) {
  const size_t big = (size_t)n * (L + 1) * (L + 1) * C * sizeof(float);
  SwLayout s{};
  s.u = 0;
  s.v = up256(big);
  s.g = s.v + up256(big);
  s.s = s.g + up256((size_t)n * C * sizeof(float));
  s.total = s.s + up256(big);
  if (sw_fused_shape(L, C, dtype)) s.total = std::max(s.total, sw_packed_bytes(L));
  return s;
}

// bf16: u, v and s in bf16 (the matrix-core path), else fp32.
template <int L>
so2_status launch_s2(const void* u, const void* v, const float* g, void* s, bool bf16, int n, int C,
                     hipStream_t stream) {
  const S2Tables<L> T = make_tables<L>();
  const int blocks = std::max(1, std::min((n + 3) / 4, 2048));
  if (bf16)
    hipLaunchKernelGGL((s2_kernel<L, uint16_t, uint16_t>), dim3(blocks), dim3(kS2Threads), 0, stream,
                       (const uint16_t*)u, (const uint16_t*)v, g, (uint16_t*)s, n, C, T);
  else
    hipLaunchKernelGGL((s2_kernel<L, float, float>), dim3(blocks), dim3(kS2Threads), 0, stream, (const float*)u,
                       (const float*)v, g, (float*)s, n, C, T);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

template <typename T>
void lin_launch(const T* in, int64_t in_stride, const T* W, float* out, int64_t out_stride, int n, int ncp, int C,
                hipStream_t stream) {
  const int64_t total = (int64_t)n * ncp * C;
  hipLaunchKernelGGL((lin_kernel<T, T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, in, in_stride,
                     W, out, out_stride, n, ncp, C);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

size_t swiglu_s2_workspace_bytes(int n_atoms, int L, int C, int dtype) {
  return sw_layout(n_atoms, L, C, dtype).total;
}

so2_status launch_swiglu_s2(uint32_t stages, const void* x, const void* w_a, const void* w_b, const void* w_g,
                            const void* w_o, float* y, int n_atoms, int L, int C, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (n_atoms == 0) return SO2_OK;
  const SwLayout lay = sw_layout(n_atoms, L, C, dtype);
  if (!workspace || workspace_bytes < lay.total || !aligned16(workspace)) return SO2_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  float* u = (float*)(ws + lay.u);
  float* v = (float*)(ws + lay.v);
  float* g = (float*)(ws + lay.g);
  void* s = ws + lay.s;
  const int nc = (L + 1) * (L + 1);
  const int64_t stride = (int64_t)nc * C;
  const bool mfma = dtype == SO2_BF16 && C == 128 && aligned16(x) && aligned16(w_a) && aligned16(w_b) &&
                    aligned16(w_g) && aligned16(w_o);
  const uint32_t all = SO2_STAGE_SW_MAPS | SO2_STAGE_SW_GRID | SO2_STAGE_SW_OUT;
  if (stages == all && mfma && sw_fused_shape(L, C, dtype)) {
    // the whole call in one kernel (after the weights' repack)
    sw_u32x4* wp = (sw_u32x4*)workspace;
    const int nthr = (3 * (L + 1) + 1) * 32 * 64;
    hipLaunchKernelGGL(sw_pack_kernel, dim3((nthr + 255) / 256), dim3(256), 0, stream, (const uint16_t*)w_a,
                       (const uint16_t*)w_b, (const uint16_t*)w_o, (const uint16_t*)w_g, wp, L);
    const uint16_t* xb = (const uint16_t*)x;
    switch (L) {
      case 0:
        launch_fused<0>(xb, wp, y, n_atoms, stream);
        break;
      case 1:
        launch_fused<1>(xb, wp, y, n_atoms, stream);
        break;
      case 2:
        launch_fused<2>(xb, wp, y, n_atoms, stream);
        break;
      case 3:
        launch_fused<3>(xb, wp, y, n_atoms, stream);
        break;
      default:
        launch_fused<4>(xb, wp, y, n_atoms, stream);
        break;
    }
    SO2_CHECK_LAUNCH();
    return SO2_OK;
  }
  if (!(stages & SO2_STAGE_SW_MAPS)) {
  } else if (mfma) {
    const unsigned nb = (unsigned)((n_atoms + kLinNodes - 1) / kLinNodes);
    hipLaunchKernelGGL((lin_mfma_kernel<2, uint16_t>), dim3(nb, L + 1), dim3(256), 0, stream, (const uint16_t*)x,
                       stride, (const uint16_t*)w_a, (const uint16_t*)w_b, (uint16_t*)u, (uint16_t*)v, stride,
                       n_atoms);
    hipLaunchKernelGGL((lin_mfma_kernel<1, float>), dim3(nb, 1), dim3(256), 0, stream, (const uint16_t*)x, stride,
                       (const uint16_t*)w_g, (const uint16_t*)w_g, g, g, (int64_t)C, n_atoms);
    SO2_CHECK_LAUNCH();
  } else if (dtype == SO2_BF16) {
    lin_launch((const uint16_t*)x, stride, (const uint16_t*)w_a, u, stride, n_atoms, nc, C, stream);
    lin_launch((const uint16_t*)x, stride, (const uint16_t*)w_b, v, stride, n_atoms, nc, C, stream);
    lin_launch((const uint16_t*)x, stride, (const uint16_t*)w_g, g, (int64_t)C, n_atoms, 1, C, stream);
    SO2_CHECK_LAUNCH();
  } else {
    lin_launch((const float*)x, stride, (const float*)w_a, u, stride, n_atoms, nc, C, stream);
    lin_launch((const float*)x, stride, (const float*)w_b, v, stride, n_atoms, nc, C, stream);
    lin_launch((const float*)x, stride, (const float*)w_g, g, (int64_t)C, n_atoms, 1, C, stream);
    SO2_CHECK_LAUNCH();
  }
  so2_status st = (stages & SO2_STAGE_SW_GRID) ? SO2_ERR_UNSUPPORTED : SO2_OK;
  if (stages & SO2_STAGE_SW_GRID) switch (L) {
    case 0:
      st = launch_s2<0>(u, v, g, s, mfma, n_atoms, C, stream);
      break;
    case 1:
      st = launch_s2<1>(u, v, g, s, mfma, n_atoms, C, stream);
      break;
    case 2:
      st = launch_s2<2>(u, v, g, s, mfma, n_atoms, C, stream);
      break;
    case 3:
      st = launch_s2<3>(u, v, g, s, mfma, n_atoms, C, stream);
      break;
    case 4:
      st = launch_s2<4>(u, v, g, s, mfma, n_atoms, C, stream);
      break;
    case 5:
      st = launch_s2<5>(u, v, g, s, mfma, n_atoms, C, stream);
      break;
    case 6:
      st = launch_s2<6>(u, v, g, s, mfma, n_atoms, C, stream);
      break;
  }
  if (st != SO2_OK) return st;
  if (!(stages & SO2_STAGE_SW_OUT)) {
  } else if (mfma) {
    const unsigned nb = (unsigned)((n_atoms + kLinNodes - 1) / kLinNodes);
    hipLaunchKernelGGL((lin_mfma_kernel<1, float>), dim3(nb, L + 1), dim3(256), 0, stream, (const uint16_t*)s,
                       stride, (const uint16_t*)w_o, (const uint16_t*)w_o, y, y, stride, n_atoms);
  } else if (dtype == SO2_BF16) {
    const int64_t total = (int64_t)n_atoms * nc * C;
    hipLaunchKernelGGL((lin_kernel<float, uint16_t>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       (const float*)s, stride, (const uint16_t*)w_o, y, stride, n_atoms, nc, C);
  } else {
    lin_launch((const float*)s, stride, (const float*)w_o, y, stride, n_atoms, nc, C, stream);
  }
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

}  // namespace so2
