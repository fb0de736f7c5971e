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
// * the grid step (s2_kernel): one wave per node, one lane per channel.  The
//   grid factorises, Y_lm(theta_i, phi_j) = Pn_lm(theta_i) T_m(phi_j) with
//   T_0 = 1, T_m = cos(m phi), T_-m = sin(m phi), so u on ring i is
//   sum_m F_m T_m(phi_j) with F_m = sum_l Pn_lm(theta_i) u_lm, and the
//   projection runs the same two sums in reverse.  Both factors have a mirror
//   symmetry (rings at +-cos(theta), meridians at +-phi) that halves each
//   sum again.  The tables Pn and T are built in LDS by each block.
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
__device__ double theta_factor(int k, double x) {
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

// s[(l, m), c] = SiLU(g_c) sum_p w_p Y_lm(r_p) u(r_p)_c v(r_p)_c, one wave per
// node (grid-stride over nodes), lanes over channels.
constexpr int kS2Threads = 256;
template <int L, typename TU, typename TS>
__global__ void __launch_bounds__(kS2Threads) __attribute__((amdgpu_waves_per_eu(L <= 3 ? 3 : 1))) s2_kernel(const TU* __restrict__ u, const TU* __restrict__ v,
                                                        const float* __restrict__ gate, TS* __restrict__ s,
                                                        int n_atoms, int C, GridArgs grid) {
  constexpr int NC = (L + 1) * (L + 1), NM = 2 * L + 1, NT = (3 * L + 2) / 2, NF = 3 * L + 1;
  constexpr int NMP = (NM + 3) & ~3;
  __shared__ __attribute__((aligned(16))) float pn[NT][NC];
  __shared__ __attribute__((aligned(16))) float tf[NF][NMP];
  __shared__ float wq[NT];
  for (int e = threadIdx.x; e < NT * NC; e += kS2Threads)
    pn[e / NC][e % NC] = (float)theta_factor(e % NC, grid.ct[e / NC]);
  for (int e = threadIdx.x; e < NF * NMP; e += kS2Threads) {
    const int j = e / NMP, mm = e % NMP - L;
    const double ph = 2.0 * kPi * j / NF;
    tf[j][e % NMP] = mm > L ? 0.0f : (float)(mm == 0 ? 1.0 : mm > 0 ? cos(mm * ph) : sin(-mm * ph));
  }
  if (threadIdx.x < NT) wq[threadIdx.x] = (float)grid.wt[threadIdx.x];
  __syncthreads();

  // One ring: the product of u and v at its NF meridians, projected onto the
  // T_m, added to g.  phi_0 = 0 (T_m = 1 for m >= 0, 0 for m < 0) stands
  // alone; phi_j and phi_{NF-j} share the cosines and have opposite sines,
  // so each pair costs one cosine sum and one sine sum per field; for even
  // NF, phi = pi stands alone too.
  auto ring_phi = [&](const float (&fu)[NM], const float (&fv)[NM], float (&g)[NM]) {
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
        const float c = tf[j][L + m], sn = tf[j][L - m];
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
        g[L + m] += tf[j][L + m] * hs;
        g[L - m] += tf[j][L - m] * hd;
      }
    }
    if constexpr (NF % 2 == 0) {
      constexpr int j = NF / 2;
      float a = 0.0f, b = 0.0f;
#pragma unroll
      for (int q = L; q < NM; ++q) {
        a += tf[j][q] * fu[q];
        b += tf[j][q] * fv[q];
      }
      const float hp = a * b;
#pragma unroll
      for (int q = L; q < NM; ++q) g[q] += tf[j][q] * hp;
    }
  };

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
        hh[k] = 0.0f;
      }
      const float z = gate[(int64_t)node * C + c];
      const float sg = z / (1.0f + expf(-z));
      // Ring pairs: rings i and NT - 1 - i have opposite cos(theta), and
      // Pn_lm(-x) = (-1)^(l+m) Pn_lm(x), so one sum over the even l + m terms
      // and one over the odd ones serve both (F = E + O on ring i, E - O on
      // its mirror); the projection back takes ga + gb or ga - gb by parity.
      for (int i = 0; i < (NT + 1) / 2; ++i) {
        const bool pair = 2 * i + 1 != NT;
        float eu[NM], ou[NM], ev[NM], ov[NM];
#pragma unroll
        for (int q = 0; q < NM; ++q) eu[q] = ou[q] = ev[q] = ov[q] = 0.0f;
#pragma unroll
        for (int l = 0; l <= L; ++l)
#pragma unroll
          for (int m = -l; m <= l; ++m) {
            const float p = pn[i][l * l + l + m];
            if (((l + m) & 1) == 0) {
              eu[m + L] += p * uu[l * l + l + m];
              ev[m + L] += p * vv[l * l + l + m];
            } else {
              ou[m + L] += p * uu[l * l + l + m];
              ov[m + L] += p * vv[l * l + l + m];
            }
          }
        float fu[NM], fv[NM], ga[NM], gb[NM];
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          fu[q] = eu[q] + ou[q];
          fv[q] = ev[q] + ov[q];
          ga[q] = gb[q] = 0.0f;
        }
        ring_phi(fu, fv, ga);
        if (pair) {
#pragma unroll
          for (int q = 0; q < NM; ++q) {
            fu[q] = eu[q] - ou[q];
            fv[q] = ev[q] - ov[q];
          }
          ring_phi(fu, fv, gb);
        }
        const float w = wq[i];
#pragma unroll
        for (int l = 0; l <= L; ++l)
#pragma unroll
          for (int m = -l; m <= l; ++m) {
            const float gq = ((l + m) & 1) == 0 ? ga[m + L] + gb[m + L] : ga[m + L] - gb[m + L];
            hh[l * l + l + m] += pn[i][l * l + l + m] * (w * gq);
          }
      }
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

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

struct SwLayout {
  size_t u, v, g, s, total;
};

SwLayout sw_layout(int n, int L, int C) {
  const size_t big = (size_t)n * (L + 1) * (L + 1) * C * sizeof(float);
  SwLayout s{};
  s.u = 0;
  s.v = up256(big);
  s.g = s.v + up256(big);
  s.s = s.g + up256((size_t)n * C * sizeof(float));
  s.total = s.s + up256(big);
  return s;
}

// bf16: u, v and s in bf16 (the matrix-core path), else fp32.
template <int L>
so2_status launch_s2(const void* u, const void* v, const float* g, void* s, bool bf16, int n, int C,
                     hipStream_t stream) {
  const GridArgs grid = make_grid(L);
  const int blocks = std::max(1, std::min((n + 3) / 4, 2048));
  if (bf16)
    hipLaunchKernelGGL((s2_kernel<L, uint16_t, uint16_t>), dim3(blocks), dim3(kS2Threads), 0, stream,
                       (const uint16_t*)u, (const uint16_t*)v, g, (uint16_t*)s, n, C, grid);
  else
    hipLaunchKernelGGL((s2_kernel<L, float, float>), dim3(blocks), dim3(kS2Threads), 0, stream, (const float*)u,
                       (const float*)v, g, (float*)s, n, C, grid);
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
  (void)dtype;
  return sw_layout(n_atoms, L, C).total;
}

so2_status launch_swiglu_s2(uint32_t stages, const void* x, const void* w_a, const void* w_b, const void* w_g,
                            const void* w_o, float* y, int n_atoms, int L, int C, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (n_atoms == 0) return SO2_OK;
  const SwLayout lay = sw_layout(n_atoms, L, C);
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
