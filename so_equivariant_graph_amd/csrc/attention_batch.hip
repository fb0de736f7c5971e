// Backward of the fused SO(2) attention forward, fp32.
//
// For a scalar loss L with upstream gradient dy = dL/dy (one row per
// target), the gradients of L with respect to the node features x, the
// positions, W_q, W_k, W_rad and the packed SO(2) weights: the derivatives
// a Conservative model takes for forces ("E2Former-V2: On-the-Fly
// Equivariant Attention with Linear Activation Memory", technical summary,
// section 4) and conservative training needs ("DPA4: Pushing the
// Accuracy-Cost Frontier of Interatomic Potentials with EMFA SO(2)
// Convolution", technical summary, section 2.2).
//
// The per-m map is the same dense map for every edge, so its three uses in
// the backward are GEMMs over a batch of edges, on the matrix cores in fp32
// (v_mfma_f32_16x16x4_f32):
//   Y  = X  B_m^T      (the forward map, recomputed),
//   dX = dY B_m        (its transpose applied to the output gradient),
//   dB_m += dY^T X     (the weight gradient, a sum over edges),
// where an edge's row X holds its rotated, gated input in the block layout
// [m = 0: (l, c)], [m = 1: (sign, l, c)], ... and B_m is W0 for m = 0 and
// [[W1, -W2], [W2, W1]] for m >= 1 (the complex product as one real matrix).
// Everything per edge that is not a GEMM (frame, Wigner-D, gate, rotations,
// softmax terms, the direction gradient) runs in per-edge kernels, one wave
// per edge.  Per-edge tensors exist only for one batch of edges at a time
// (a fixed capacity set from the target count), so memory is linear in the
// atom count plus a constant; only the softmax statistics per (target, head)
// and the head sums Sbar below live across batches:
//   statistics  running max M and normaliser sum_j u_ij exp(z_ij - M);
//   pass 1      per edge v_ij = D^T Y_ij and s_ij^h = <dy_i, v_ij> over the
//               channels of head h; Sbar_i^h = sum_j a_ij^h s_ij^h;
//   pass 2      per edge, again v and s, then
//     dL/dz^h = a^h (s^h - Sbar^h),  dL/du = sum_h abar^h (s^h - Sbar^h)
//     (abar = a / u = exp(z - M) / normaliser),
//     dv = a (.) dy_i,  dyt = D dv,  then the GEMMs dB_m += dyt^T xt and
//     dxt = map^T(dyt),  and per edge
//     dg[c] = sum_(l,m) dxt xh (xh = D x_j before the gate),
//     dx_j += D^T (dxt (.) g),  dW_rad += phi dg (a GEMM over the batch),
//     d|r| = sum_c dg[c] dg_c/d|r| + dL/du du/d|r|,
//     direction: a rotation w of the edge direction r_hat -> r_hat + w x
//     r_hat is a frame R exp(-[w]x), so D -> D (I - sum_a w_a J_a) with J_a
//     the rotation generators in the real harmonic basis, and
//       dL/dw_a = <dv, J_a v> - <dxt (.) g, D J_a x_j>;
//     the direction gradient is (dL/dw) x r_hat, so
//       dL/dr = (dL/dw) x r_hat / |r| + d|r| r_hat,
//     added to dpos[j] and taken from dpos[i];
//     dq_i += dz k_j / sqrt(d), dk_j += dz q_i / sqrt(d).
// When every edge fits one batch, pass 2 reuses pass 1's batch; otherwise
// it recomputes each batch (forward map included), the last batch of pass
// 1 first.  A last kernel takes dq and dk through the projections of the
// l = 0 slice: dx[., 0, .] += dq W_q^T + dk W_k^T, dW_q = x0^T dq,
// dW_k = x0^T dk.  Sums that several edges add to (dx of sources, dpos, dq,
// dk, Sbar, the weight gradients) use fp32 atomics, so their summation
// order varies between runs.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "wigner.h"

namespace so2 {

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kLane = 64;       // per-edge and per-target kernels: one wave per block
constexpr int kMaxHeadsB = 256;  // heads (and focus streams), per-lane loops of stride 64
constexpr int kScal = 12;       // per-edge scalars (EdgeBufs::sc)
constexpr int kGridCap = 16384; // blocks of a grid-stride per-edge launch

// ---------------------------------------------------------------- layouts

// Width of block m of an edge row: (L+1) C for m = 0, 2 (L+1-m) C for m >= 1.
__host__ __device__ inline int blk_width(int L, int C, int m) { return (m == 0 ? 1 : 2) * (L + 1 - m) * C; }
// Column of block m in an edge row.
__host__ __device__ inline int blk_off(int L, int C, int m) {
  int off = 0;
  for (int q = 0; q < m; ++q) off += blk_width(L, C, q);
  return off;
}
// Offset of B_m in the B array: F stream matrices of (blk_width / F)^2
// floats each, row-major [out][in] (F = 1: one matrix per block).
__host__ __device__ inline int64_t bmat_off(int L, int C, int m, int F = 1) {
  int64_t off = 0;
  for (int q = 0; q < m; ++q) off += (int64_t)(blk_width(L, C, q) / F) * (blk_width(L, C, q) / F) * F;
  return off;
}
// Column of component (l, mm) (|mm| <= l) for channel 0: block |mm|, sign
// half for mm < 0, degree l - |mm| inside it.
__device__ inline int comp_col(int L, int C, int l, int mm) {
  const int m = mm < 0 ? -mm : mm;
  return blk_off(L, C, m) + (mm < 0 ? (L + 1 - m) * C : 0) + (l - m) * C;
}

// Per-edge tensors of one batch (capacity cap edges), fp32.
struct EdgeBufs {
  float* xt;   // [cap][nc C]  xt, then dxt (block layout)
  float* yt;   // [cap][nc C]  yt, then dyt (block layout)
  float* D;    // [cap][wig_total(L)]
  float* g;    // [cap][C]  radial gate
  float* gp;   // [cap][C]  d gate / d|r|
  float* dg;   // [cap][C]  dL/d gate
  float* phi;  // [cap][K]  radial basis (times u with the envelope flag)
  float* a;    // [cap][H]  softmax weight u exp(z - M) / normaliser
  float* ab;   // [cap][H]  a / u
  float* sc;   // [cap][kScal]: |r|, u, du/d|r|, r_hat (3), dL/du, <dv, J_a v> (3)
  int32_t* tgt;  // [cap]
};

struct BatchParams {
  const float* pos;
  float* y;           // forward: [n_targets][(L+1)^2][C]
  const void* w_logit;  // [K][H] radial logit bias, or null
  const void* w_focus;  // [C] focus scores when n_focus > 1
  int32_t m_max, n_focus;
  const int32_t* row_ptr;
  const int32_t* col;
  const void* x;
  const void* w_rad;
  const float* dy;
  const float* q;     // [n_atoms][C]
  const float* k;     // [n_atoms][C]
  const float* gen;   // [3][wig_total(L)] rotation generators
  float* smax;  // [n_targets][H]
  float* sinv;  // [n_targets][H] 1 / normaliser (0 if it is 0)
  float* sbar;        // [n_targets][H]
  float* dq;          // [n_targets][C]
  float* dk;          // [n_atoms][C]
  float* dx;
  float* dpos;
  EdgeBufs b;
  int64_t e0;  // first edge of the batch (CSR index)
  int32_t nb;  // edges in the batch
  int32_t n_targets, C, H, K, p;
  float cutoff;
  uint32_t flags;
  int32_t periodic;
  float box[3];
};

// Compiler-only barrier (no instruction): LDS reads of the Wigner-D and
// generator blocks are not moved across it, so they are re-read per degree
// and channel instead of being hoisted into registers for the whole edge.
__device__ inline void keep_order() { asm volatile("" ::: "memory"); }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Radial logit bias of head h for an edge of length rho: sum_k phi_k(rho)
// w_logit[k][h] with the gate's Gaussian basis (0 without the bias).  sphi,
// if given, holds phi_0 .. phi_63 of this edge.
template <typename T>
__device__ inline float logit_bias(const BatchParams& P, int h, float rho, const float* sphi) {
  if (!P.w_logit) return 0.0f;
  const float step = P.cutoff / (float)(P.K - 1);
  const float inv2s2 = 1.0f / (2.0f * step * step);
  float b = 0.0f;
  for (int kk = 0; kk < P.K; ++kk) {
    float ph;
    if (sphi && kk < 64) {
      ph = sphi[kk];
    } else {
      const float dr = rho - step * (float)kk;
      ph = expf(-dr * dr * inv2s2);
    }
    b += ph * load_as_float((const T*)P.w_logit, (int64_t)kk * P.H + h);
  }
  return b;
}

// ---------------------------------------------------------------- statistics

// One wave per target: for every head the running max of the logits and the
// normaliser sum_j u_ij exp(z_ij - max), over the target's edges in order.
// Lane l keeps heads l, l + 64, ...
constexpr int kHeadsPerLane = kMaxHeadsB / kLane;
template <typename T>
__global__ void __launch_bounds__(kLane) batch_stats_kernel(BatchParams P) {
  __shared__ float zs[kMaxHeadsB];
  const int lane = threadIdx.x;
  const int C = P.C, H = P.H, d = C / H;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  for (int i = blockIdx.x; i < P.n_targets; i += gridDim.x) {
    float m[kHeadsPerLane], sum[kHeadsPerLane];
#pragma unroll
    for (int r = 0; r < kHeadsPerLane; ++r) {
      m[r] = -INFINITY;
      sum[r] = 0.0f;
    }
    for (int e = P.row_ptr[i]; e < P.row_ptr[i + 1]; ++e) {
      const int j = P.col[e];
      for (int h = lane; h < H; h += kLane) zs[h] = 0.0f;
      __syncthreads();
      for (int c = lane; c < C; c += kLane) atomicAdd(&zs[c / d], P.q[(int64_t)i * C + c] * P.k[(int64_t)j * C + c]);
      __syncthreads();
      if (lane < H) {
        const EdgeGeo geo = edge_geometry(P.pos, i, j, P.periodic, P.box, P.cutoff);
        const float u = envelope_u(geo.s, geo.t, P.p);
#pragma unroll
        for (int r = 0; r < kHeadsPerLane; ++r) {
          const int h = lane + kLane * r;
          if (h >= H) break;
          const float z = zs[h] * inv_sqrt_d + logit_bias<T>(P, h, geo.rho, nullptr);
          if (z > m[r]) {
            sum[r] = sum[r] * expf(m[r] - z) + u;
            m[r] = z;
          } else {
            sum[r] += u * expf(z - m[r]);
          }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < kHeadsPerLane; ++r) {
      const int h = lane + kLane * r;
      if (h < H) {
        P.smax[(int64_t)i * H + h] = m[r];
        P.sinv[(int64_t)i * H + h] = sum[r] > 0.0f ? 1.0f / sum[r] : 0.0f;
      }
    }
  }
}

// ---------------------------------------------------------------- per-edge kernels

// D^0 .. D^L of the edge into LDS (sD, wig_total(L) floats) from its frame:
// D^1 directly, then one degree at a time over the lanes.
template <int L>
__device__ inline void edge_wigner(const float* rh, float* sD) {
  const int lane = threadIdx.x;
  float R[9], D1[9];
  edge_frame(rh[0], rh[1], rh[2], R);
  wigner_l1(R, D1);
  if (lane == 0) sD[0] = 1.0f;
  if (L >= 1 && lane < 9) sD[wig_offset(1) + lane] = D1[lane];
  __syncthreads();
#pragma unroll
  for (int l = 2; l <= L; ++l) {
    const int n = 2 * l + 1;
    for (int q = lane; q < n * n; q += kLane)
      sD[wig_offset(l) + q] = wigner_entry(l, q / n - l, q % n - l, sD + wig_offset(1), sD + wig_offset(l - 1));
    __syncthreads();
  }
}

// Largest target i with row_ptr[i] <= e (the target of CSR edge e).
__device__ inline int edge_target(const int32_t* row_ptr, int n_targets, int64_t e) {
  int lo = 0, hi = n_targets;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (row_ptr[mid] <= e) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The target of every edge of the batch, one thread per edge (the per-edge
// kernels read it instead of searching row_ptr with a whole wave per edge).
__global__ void __launch_bounds__(256) batch_targets_kernel(BatchParams P) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < P.nb) P.b.tgt[e] = edge_target(P.row_ptr, P.n_targets, P.e0 + e);
}

// Pass-1 preparation of every edge of the batch (its target from
// batch_targets_kernel): geometry, frame,
// Wigner-D, radial basis, gate and its |r| derivative, softmax weights, and
// xt = g (.) D x_j in the block layout.
template <int L, typename T>
__global__ void __launch_bounds__(kLane) __attribute__((amdgpu_waves_per_eu(4))) bwd_prep_kernel(BatchParams P) {
  constexpr int nw = wig_total(L);
  constexpr int nc = n_comp(L);
  __shared__ float sD[nw];
  __shared__ float sphi[64];
  __shared__ float zs[kMaxHeadsB];
  const int lane = threadIdx.x;
  const int C = P.C, H = P.H, K = P.K, d = C / H;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  const float rc = P.cutoff;
  const bool radial = !(P.flags & SO2_FLAG_NO_RADIAL);
  const bool rbf_env = (P.flags & SO2_FLAG_RBF_ENVELOPE) != 0;
  const float mu_step = rc / (float)(K - 1);
  const float inv2s2 = 1.0f / (2.0f * mu_step * mu_step);
  const T* x = (const T*)P.x;
  const T* wr = (const T*)P.w_rad;
  const EdgeBufs& B = P.b;
  for (int e = blockIdx.x; e < P.nb; e += gridDim.x) {
    const int64_t ge = P.e0 + e;
    const int i = B.tgt[e];
    const int j = P.col[ge];
    const EdgeGeo geo = edge_geometry(P.pos, i, j, P.periodic, P.box, rc);
    const float rho = geo.rho;
    const float u = envelope_u(geo.s, geo.t, P.p);
    const float dudr = envelope_du(geo.s, geo.t, P.p) / rc;
    const float inv = rho > 0.0f ? 1.0f / rho : 0.0f;
    const float rh[3] = {geo.r[0] * inv, geo.r[1] * inv, geo.r[2] * inv};
    edge_wigner<L>(rh, sD);
    for (int q = lane; q < nw; q += kLane) B.D[(int64_t)e * nw + q] = sD[q];
    for (int kk = lane; kk < K; kk += kLane) {
      const float dr = rho - mu_step * (float)kk;
      const float ph = expf(-dr * dr * inv2s2);
      if (kk < 64) sphi[kk] = ph;
      if (B.phi) B.phi[(int64_t)e * K + kk] = rbf_env ? ph * u : ph;
    }
    for (int h = lane; h < H; h += kLane) zs[h] = 0.0f;
    if (lane == 0) {
      if (B.sc) {
        float* sc = B.sc + (int64_t)e * kScal;
        sc[0] = rho;
        sc[1] = u;
        sc[2] = dudr;
        sc[3] = rh[0];
        sc[4] = rh[1];
        sc[5] = rh[2];
      }
    }
    __syncthreads();
    float* xte = B.xt + (int64_t)e * nc * C;
    for (int c = lane; c < C; c += kLane) {
      float g = 1.0f, gp = 0.0f;
      if (radial) {
        float g0 = 0.0f, gd = 0.0f;
        for (int kk = 0; kk < K; ++kk) {
          const float dr = rho - mu_step * (float)kk;
          const float ph = kk < 64 ? sphi[kk] : expf(-dr * dr * inv2s2);
          const float w = load_as_float(wr, (int64_t)kk * C + c);
          g0 += ph * w;
          gd += -dr * 2.0f * inv2s2 * ph * w;
        }
        g = rbf_env ? g0 * u : g0;
        gp = rbf_env ? gd * u + g0 * dudr : gd;
      }
      if (B.g) {
        B.g[(int64_t)e * C + c] = g;
        B.gp[(int64_t)e * C + c] = gp;
      }
      atomicAdd(&zs[c / d], P.q[(int64_t)i * C + c] * P.k[(int64_t)j * C + c]);
      const T* xj = x + (int64_t)j * nc * C + c;
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        keep_order();
        const int n = 2 * l + 1;
        float xv[2 * L + 1];
#pragma unroll
        for (int b = 0; b < n; ++b) xv[b] = load_as_float(xj, (int64_t)(l * l + b) * C);
        const float* Dl = sD + wig_offset(l);
#pragma unroll
        for (int mr = 0; mr < n; ++mr) {
          // orders past m_max have no block (their map output is 0)
          if (mr - l > P.m_max || l - mr > P.m_max) continue;
          float v = 0.0f;
#pragma unroll
          for (int b = 0; b < n; ++b) v += Dl[mr * n + b] * xv[b];
          xte[comp_col(L, C, l, mr - l) + c] = g * v;
        }
      }
    }
    __syncthreads();
    for (int h = lane; h < H; h += kLane) {
      const float z = zs[h] * inv_sqrt_d + logit_bias<T>(P, h, rho, sphi);
      const float ab = expf(z - P.smax[(int64_t)i * H + h]) * P.sinv[(int64_t)i * H + h];
      B.ab[(int64_t)e * H + h] = ab;
      B.a[(int64_t)e * H + h] = u * ab;
    }
    __syncthreads();
  }
}

// v = D^T yt for degree l of one channel: yt read from the block layout.
template <int L, int l>
__device__ inline void rotate_back(const float* sD, const float* yte, int C, int c, float (&v)[2 * L + 1]) {
  constexpr int n = 2 * l + 1;
  float yv[n];
#pragma unroll
  for (int r = 0; r < n; ++r) yv[r] = yte[comp_col(L, C, l, r - l) + c];
  const float* Dl = sD + wig_offset(l);
#pragma unroll
  for (int b = 0; b < n; ++b) {
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < n; ++r) s += Dl[r * n + b] * yv[r];
    v[b] = s;
  }
}

// <dy_i, v> over degree l of one channel.
template <int L, int l>
__device__ inline float head_part(const float* sD, const float* yte, const float* dyi, int C, int c) {
  keep_order();
  float v[2 * L + 1];
  rotate_back<L, l>(sD, yte, C, c, v);
  float s = 0.0f;
#pragma unroll
  for (int b = 0; b < 2 * l + 1; ++b) s += dyi[(int64_t)(l * l + b) * C + c] * v[b];
  return s;
}

template <int L, int l>
__device__ inline float head_sum(const float* sD, const float* yte, const float* dyi, int C, int c) {
  if constexpr (l > L) return 0.0f;
  else return head_part<L, l>(sD, yte, dyi, C, c) + head_sum<L, l + 1>(sD, yte, dyi, C, c);
}

// Pass 1: s^h of every edge and Sbar_i^h += a^h s^h.
template <int L>
__global__ void __launch_bounds__(kLane) __attribute__((amdgpu_waves_per_eu(4))) bwd_sbar_kernel(BatchParams P) {
  constexpr int nw = wig_total(L);
  constexpr int nc = n_comp(L);
  __shared__ float sD[nw];
  __shared__ float ss[kMaxHeadsB];
  const int lane = threadIdx.x;
  const int C = P.C, H = P.H, d = C / H;
  const EdgeBufs& B = P.b;
  for (int e = blockIdx.x; e < P.nb; e += gridDim.x) {
    const int i = B.tgt[e];
    for (int q = lane; q < nw; q += kLane) sD[q] = B.D[(int64_t)e * nw + q];
    for (int h = lane; h < H; h += kLane) ss[h] = 0.0f;
    __syncthreads();
    const float* yte = B.yt + (int64_t)e * nc * C;
    const float* dyi = P.dy + (int64_t)i * nc * C;
    for (int c = lane; c < C; c += kLane) atomicAdd(&ss[c / d], head_sum<L, 0>(sD, yte, dyi, C, c));
    __syncthreads();
    for (int h = lane; h < H; h += kLane) atomicAdd(P.sbar + (int64_t)i * H + h, B.a[(int64_t)e * H + h] * ss[h]);
    __syncthreads();
  }
}

// Degree l of one channel in pass 2: dv = a dy_i, <dv, J_a v> into dir,
// dyt = D dv written over yt.
template <int L, int l>
__device__ inline void dyt_degree(const float* sD, const float* sJ, float* yte, const float* dyi, int C, int c,
                                  float av, float (&dir)[3]) {
  constexpr int n = 2 * l + 1;
  constexpr int nw = wig_total(L);
  keep_order();
  float v[2 * L + 1];
  rotate_back<L, l>(sD, yte, C, c, v);
  float dv[n];
#pragma unroll
  for (int b = 0; b < n; ++b) dv[b] = av * dyi[(int64_t)(l * l + b) * C + c];
#pragma unroll
  for (int ax = 0; ax < 3; ++ax) {
    keep_order();
    const float* Jl = sJ + ax * nw + wig_offset(l);
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < n; ++m) {
      float jv = 0.0f;
#pragma unroll
      for (int b = 0; b < n; ++b) jv += Jl[m * n + b] * v[b];
      s += dv[m] * jv;
    }
    dir[ax] += s;
  }
  keep_order();
  const float* Dl = sD + wig_offset(l);
#pragma unroll
  for (int r = 0; r < n; ++r) {
    float s = 0.0f;
#pragma unroll
    for (int b = 0; b < n; ++b) s += Dl[r * n + b] * dv[b];
    yte[comp_col(L, C, l, r - l) + c] = s;
  }
}

template <int L, int l>
__device__ inline void dyt_all(const float* sD, const float* sJ, float* yte, const float* dyi, int C, int c, float av,
                               float (&dir)[3]) {
  if constexpr (l <= L) {
    dyt_degree<L, l>(sD, sJ, yte, dyi, C, c, av, dir);
    dyt_all<L, l + 1>(sD, sJ, yte, dyi, C, c, av, dir);
  }
}

// Pass 2, first half: s^h again, dL/dz, dL/du, dyt (over yt), the first
// direction term, dq and dk.
template <int L>
__global__ void __launch_bounds__(kLane) __attribute__((amdgpu_waves_per_eu(4))) bwd_dyt_kernel(BatchParams P) {
  constexpr int nw = wig_total(L);
  constexpr int nc = n_comp(L);
  __shared__ float sD[nw];
  __shared__ float sJ[3 * nw];
  __shared__ float ss[kMaxHeadsB];
  __shared__ float sdz[kMaxHeadsB];
  __shared__ float sa[kMaxHeadsB];
  const int lane = threadIdx.x;
  const int C = P.C, H = P.H, d = C / H;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  const EdgeBufs& B = P.b;
  for (int q = lane; q < 3 * nw; q += kLane) sJ[q] = P.gen[q];
  for (int e = blockIdx.x; e < P.nb; e += gridDim.x) {
    const int i = B.tgt[e];
    const int j = P.col[P.e0 + e];
    for (int q = lane; q < nw; q += kLane) sD[q] = B.D[(int64_t)e * nw + q];
    for (int h = lane; h < H; h += kLane) ss[h] = 0.0f;
    __syncthreads();
    float* yte = B.yt + (int64_t)e * nc * C;
    const float* dyi = P.dy + (int64_t)i * nc * C;
    for (int c = lane; c < C; c += kLane) atomicAdd(&ss[c / d], head_sum<L, 0>(sD, yte, dyi, C, c));
    __syncthreads();
    float du = 0.0f;
    for (int h = lane; h < H; h += kLane) {
      const float diff = ss[h] - P.sbar[(int64_t)i * H + h];
      const float a = B.a[(int64_t)e * H + h];
      sdz[h] = a * diff * inv_sqrt_d;
      sa[h] = a;
      du += B.ab[(int64_t)e * H + h] * diff;
    }
    du = wave_sum(du);
    __syncthreads();
    float dir[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll 1
    for (int c = lane; c < C; c += kLane) {
      const int h = c / d;
      dyt_all<L, 0>(sD, sJ, yte, dyi, C, c, sa[h], dir);
      atomicAdd(P.dq + (int64_t)i * C + c, sdz[h] * P.k[(int64_t)j * C + c]);
      atomicAdd(P.dk + (int64_t)j * C + c, sdz[h] * P.q[(int64_t)i * C + c]);
    }
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) dir[ax] = wave_sum(dir[ax]);
    if (lane == 0) {
      float* sc = B.sc + (int64_t)e * kScal;
      sc[6] = du;
      sc[7] = dir[0];
      sc[8] = dir[1];
      sc[9] = dir[2];
    }
    __syncthreads();
  }
}

// Degree l of one channel in the last per-edge step: dg, dx_j, the second
// direction term.
template <int L, int l, typename T>
__device__ inline void final_degree(const float* sD, const float* sDJ, const float* xte, const T* xj, float* dxj,
                                    int C, int c, float g, float& dg, float (&dir)[3]) {
  constexpr int n = 2 * l + 1;
  constexpr int nw = wig_total(L);
  keep_order();
  float xv[n], gx[n];
#pragma unroll
  for (int b = 0; b < n; ++b) xv[b] = load_as_float(xj, (int64_t)(l * l + b) * C + c);
  const float* Dl = sD + wig_offset(l);
#pragma unroll
  for (int r = 0; r < n; ++r) {
    const float dxt = xte[comp_col(L, C, l, r - l) + c];
    float xh = 0.0f;
#pragma unroll
    for (int b = 0; b < n; ++b) xh += Dl[r * n + b] * xv[b];
    dg += dxt * xh;
    gx[r] = dxt * g;
  }
#pragma unroll
  for (int ax = 0; ax < 3; ++ax) {
    keep_order();
    const float* R = sDJ + ax * nw + wig_offset(l);
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < n; ++r) {
      float t = 0.0f;
#pragma unroll
      for (int b = 0; b < n; ++b) t += R[r * n + b] * xv[b];
      s += gx[r] * t;
    }
    dir[ax] += s;
  }
  keep_order();
#pragma unroll
  for (int b = 0; b < n; ++b) {
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < n; ++r) s += Dl[r * n + b] * gx[r];
    atomicAdd(dxj + (int64_t)(l * l + b) * C + c, s);
  }
}

template <int L, int l, typename T>
__device__ inline void final_all(const float* sD, const float* sDJ, const float* xte, const T* xj, float* dxj, int C,
                                 int c, float g, float& dg, float (&dir)[3]) {
  if constexpr (l <= L) {
    final_degree<L, l, T>(sD, sDJ, xte, xj, dxj, C, c, g, dg, dir);
    final_all<L, l + 1, T>(sD, sDJ, xte, xj, dxj, C, c, g, dg, dir);
  }
}

// Pass 2, second half (after dxt = map^T(dyt) is in the xt buffer): dg,
// dx_j, the radial and direction parts of the edge vector's gradient.
template <int L, typename T>
__global__ void __launch_bounds__(kLane) __attribute__((amdgpu_waves_per_eu(4))) bwd_final_kernel(BatchParams P) {
  constexpr int nw = wig_total(L);
  constexpr int nc = n_comp(L);
  __shared__ float sD[nw];
  __shared__ float sJ[3 * nw];
  __shared__ float sDJ[3 * nw];
  const int lane = threadIdx.x;
  const int C = P.C;
  const T* x = (const T*)P.x;
  const EdgeBufs& B = P.b;
  for (int q = lane; q < 3 * nw; q += kLane) sJ[q] = P.gen[q];
  for (int e = blockIdx.x; e < P.nb; e += gridDim.x) {
    const int i = B.tgt[e];
    const int j = P.col[P.e0 + e];
    for (int q = lane; q < nw; q += kLane) sD[q] = B.D[(int64_t)e * nw + q];
    __syncthreads();
    // D J_a per degree
    for (int q = lane; q < 3 * nw; q += kLane) {
      const int ax = q / nw, r = q % nw;
      int l = 0;
      while (wig_offset(l + 1) <= r) ++l;
      const int n = 2 * l + 1, o = r - wig_offset(l), m = o / n, mp = o % n;
      const float* Dl = sD + wig_offset(l) + m * n;
      const float* Jl = sJ + ax * nw + wig_offset(l);
      float acc = 0.0f;
      for (int b = 0; b < n; ++b) acc += Dl[b] * Jl[b * n + mp];
      sDJ[q] = acc;
    }
    __syncthreads();
    const float* xte = B.xt + (int64_t)e * nc * C;
    const T* xj = x + (int64_t)j * nc * C;
    float* dxj = P.dx + (int64_t)j * nc * C;
    float dir[3] = {0.0f, 0.0f, 0.0f};
    float rad = 0.0f;
#pragma unroll 1
    for (int c = lane; c < C; c += kLane) {
      float dg = 0.0f;
      final_all<L, 0, T>(sD, sDJ, xte, xj, dxj, C, c, B.g[(int64_t)e * C + c], dg, dir);
      B.dg[(int64_t)e * C + c] = dg;
      rad += dg * B.gp[(int64_t)e * C + c];
    }
    rad = wave_sum(rad);
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) dir[ax] = wave_sum(dir[ax]);
    if (lane == 0) {
      const float* sc = B.sc + (int64_t)e * kScal;
      const float rho = sc[0], dudr = sc[2], rx = sc[3], ry = sc[4], rz = sc[5];
      const float drho = rad + sc[6] * dudr;
      const float w0 = sc[7] - dir[0], w1 = sc[8] - dir[1], w2 = sc[9] - dir[2];
      const float inv = rho > 0.0f ? 1.0f / rho : 0.0f;
      // (dL/dw) x r_hat / |r| + d|r| r_hat
      const float gx = (w1 * rz - w2 * ry) * inv + drho * rx;
      const float gy = (w2 * rx - w0 * rz) * inv + drho * ry;
      const float gz = (w0 * ry - w1 * rx) * inv + drho * rz;
      atomicAdd(P.dpos + 3 * (int64_t)j + 0, gx);
      atomicAdd(P.dpos + 3 * (int64_t)j + 1, gy);
      atomicAdd(P.dpos + 3 * (int64_t)j + 2, gz);
      atomicAdd(P.dpos + 3 * (int64_t)i + 0, -gx);
      atomicAdd(P.dpos + 3 * (int64_t)i + 1, -gy);
      atomicAdd(P.dpos + 3 * (int64_t)i + 2, -gz);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- forward

// Degree l of one channel of the forward message: v = D^T ytilde over the
// orders up to m_max (the others have no block), times the edge's weight w,
// into the natural layout [(L+1)^2][C].
template <int L, int l>
__device__ inline void fwd_degree(const float* sD, const float* yte, float* out, int C, int c, int m_max, float w) {
  if constexpr (l <= L) {
    constexpr int n = 2 * l + 1;
    keep_order();
    float yv[n];
#pragma unroll
    for (int r = 0; r < n; ++r) yv[r] = (r - l <= m_max && l - r <= m_max) ? yte[comp_col(L, C, l, r - l) + c] : 0.0f;
    const float* Dl = sD + wig_offset(l);
#pragma unroll
    for (int b = 0; b < n; ++b) {
      float s = 0.0f;
#pragma unroll
      for (int r = 0; r < n; ++r) s += Dl[r * n + b] * yv[r];
      out[(int64_t)(l * l + b) * C + c] = w * s;
    }
    fwd_degree<L, l + 1>(sD, yte, out, C, c, m_max, w);
  }
}

// Forward, per edge once the per-m maps are in yt: the cross-focus softmax
// (n_focus > 1: pi_f = softmax_f(sum_{c in f} w_focus[c] ytilde[(0,0), c])),
// the rotation back and the softmax weights; the edge's message
// a^h pi_f D^T ytilde goes over its xt row, which the map has consumed.
template <int L, typename T>
__global__ void __launch_bounds__(kLane) __attribute__((amdgpu_waves_per_eu(4))) fwd_finish_kernel(BatchParams P) {
  constexpr int nw = wig_total(L);
  constexpr int nc = n_comp(L);
  __shared__ float sD[nw];
  __shared__ float sa[kMaxHeadsB];
  __shared__ float sp[kMaxHeadsB];
  const int lane = threadIdx.x;
  const int C = P.C, H = P.H, d = C / H, F = P.n_focus, cf = C / F;
  const EdgeBufs& B = P.b;
  for (int e = blockIdx.x; e < P.nb; e += gridDim.x) {
    for (int q = lane; q < nw; q += kLane) sD[q] = B.D[(int64_t)e * nw + q];
    for (int h = lane; h < H; h += kLane) sa[h] = B.a[(int64_t)e * H + h];
    const float* yte = B.yt + (int64_t)e * nc * C;
    if (F > 1) {
      for (int f = lane; f < F; f += kLane) sp[f] = 0.0f;
      __syncthreads();
      // ytilde[(0,0), c] is column c of the m = 0 block
      for (int c = lane; c < C; c += kLane) atomicAdd(&sp[c / cf], load_as_float((const T*)P.w_focus, c) * yte[c]);
      __syncthreads();
      if (lane == 0) {
        float mx = -INFINITY;
        for (int f = 0; f < F; ++f) mx = fmaxf(mx, sp[f]);
        float sum = 0.0f;
        for (int f = 0; f < F; ++f) {
          sp[f] = expf(sp[f] - mx);
          sum += sp[f];
        }
        const float inv = 1.0f / sum;
        for (int f = 0; f < F; ++f) sp[f] *= inv;
      }
    }
    __syncthreads();
    float* out = B.xt + (int64_t)e * nc * C;
#pragma unroll 1
    for (int c = lane; c < C; c += kLane) {
      const float w = sa[c / d] * (F > 1 ? sp[c / cf] : 1.0f);
      fwd_degree<L, 0>(sD, yte, out, C, c, P.m_max, w);
    }
    __syncthreads();
  }
}

// Degree l of one channel, accumulated: acc[(l, b)] += w (D^T ytilde)[b]
// over the orders up to m_max.
template <int L, int l>
__device__ inline void fwd_degree_acc(const float* sD, const float* yte, float (&acc)[n_comp(L)], int C, int c,
                                      int m_max, float w) {
  if constexpr (l <= L) {
    constexpr int n = 2 * l + 1;
    keep_order();
    float yv[n];
#pragma unroll
    for (int r = 0; r < n; ++r) yv[r] = (r - l <= m_max && l - r <= m_max) ? yte[comp_col(L, C, l, r - l) + c] : 0.0f;
    const float* Dl = sD + wig_offset(l);
#pragma unroll
    for (int b = 0; b < n; ++b) {
      float s = 0.0f;
#pragma unroll
      for (int r = 0; r < n; ++r) s += Dl[r * n + b] * yv[r];
      acc[l * l + b] += w * s;
    }
    fwd_degree_acc<L, l + 1>(sD, yte, acc, C, c, m_max, w);
  }
}

// Forward for C <= 128, one workgroup of 128 threads per target of the
// batch, one channel per thread: the target's edges in order (cross-focus
// softmax, rotation back, weights), the channel's sums kept in registers,
// then y[t] += the sums once.  Replaces the finishing kernel's per-edge
// messages and their per-target sum, so the messages never go through
// memory.
constexpr int kTargetThreads = 128;
template <int L, typename T>
__global__ void __launch_bounds__(kTargetThreads) fwd_target_kernel(BatchParams P) {
  constexpr int nw = wig_total(L);
  constexpr int nc = n_comp(L);
  __shared__ float sD[nw];
  __shared__ float sa[kMaxHeadsB];
  __shared__ float sp[kMaxHeadsB];
  const int tid = threadIdx.x;
  const int C = P.C, H = P.H, d = C / H, F = P.n_focus, cf = C / F;
  const EdgeBufs& B = P.b;
  const int t0 = B.tgt[0], t1 = B.tgt[P.nb - 1];
  const int c = tid;
  for (int t = t0 + blockIdx.x; t <= t1; t += gridDim.x) {
    const int64_t lo = max((int64_t)P.row_ptr[t], P.e0) - P.e0;
    const int64_t hi = min((int64_t)P.row_ptr[t + 1], P.e0 + P.nb) - P.e0;
    if (lo >= hi) continue;
    float acc[nc];
#pragma unroll
    for (int q = 0; q < nc; ++q) acc[q] = 0.0f;
    for (int64_t e = lo; e < hi; ++e) {
      __syncthreads();  // the previous edge's LDS reads are done
      for (int q = tid; q < nw; q += kTargetThreads) sD[q] = B.D[e * nw + q];
      for (int h = tid; h < H; h += kTargetThreads) sa[h] = B.a[e * H + h];
      const float* yte = B.yt + e * nc * C;
      if (F > 1) {
        for (int f = tid; f < F; f += kTargetThreads) sp[f] = 0.0f;
        __syncthreads();
        if (c < C) atomicAdd(&sp[c / cf], load_as_float((const T*)P.w_focus, c) * yte[c]);
        __syncthreads();
        if (tid == 0) {
          float mx = -INFINITY;
          for (int f = 0; f < F; ++f) mx = fmaxf(mx, sp[f]);
          float sum = 0.0f;
          for (int f = 0; f < F; ++f) {
            sp[f] = expf(sp[f] - mx);
            sum += sp[f];
          }
          const float inv = 1.0f / sum;
          for (int f = 0; f < F; ++f) sp[f] *= inv;
        }
      }
      __syncthreads();
      if (c < C) fwd_degree_acc<L, 0>(sD, yte, acc, C, c, P.m_max, sa[c / d] * (F > 1 ? sp[c / cf] : 1.0f));
    }
    if (c < C) {
      float* yt = P.y + (int64_t)t * nc * C + c;
#pragma unroll
      for (int q = 0; q < nc; ++q) yt[(int64_t)q * C] += acc[q];
    }
  }
}

// y[t] += the messages of target t's edges in this batch, in edge order
// (targets split between batches get one partial sum per batch).
__global__ void __launch_bounds__(256) fwd_reduce_kernel(BatchParams P, int ncc) {
  const int t0 = P.b.tgt[0], t1 = P.b.tgt[P.nb - 1];
  for (int t = t0 + blockIdx.x; t <= t1; t += gridDim.x) {
    const int64_t lo = max((int64_t)P.row_ptr[t], P.e0) - P.e0;
    const int64_t hi = min((int64_t)P.row_ptr[t + 1], P.e0 + P.nb) - P.e0;
    if (lo >= hi) continue;
    float* yt = P.y + (int64_t)t * ncc;
    for (int q = threadIdx.x; q < ncc; q += blockDim.x) {
      float acc = 0.0f;
      for (int64_t e = lo; e < hi; ++e) acc += P.b.xt[e * ncc + q];
      yt[q] += acc;
    }
  }
}

// ---------------------------------------------------------------- fp32 GEMM

// C (+)= A B on the matrix cores (v_mfma_f32_16x16x4_f32), fp32 throughout.
//   A(m, k) = A[m lda + k]      (AT = false)  or A[k lda + m] (AT = true)
//   B(k, n) = B[n ldb + k]      (BT = true)   or B[k ldb + n] (BT = false)
// 128 x 128 tiles of C per workgroup (4 waves, 64 x 64 each: 16 MFMA tiles
// of 16 x 16), K in steps of kGemmK staged through LDS; the next step's global
// loads go to registers while the current step's MFMAs run.  blockIdx.z
// splits K into ranges of k_split.  Mode: store (C = AB, one workgroup per
// tile) or atomic (C += AB, fp32 atomics, any number of K ranges).
struct GemmArgs {
  const float* A;
  const float* B;
  float* Cm;
  int M, N, K;
  int64_t lda, ldb, ldc;
  int k_split;  // K range per blockIdx.z
  int atomic;
  // column maps of A (AT = false) and C: index x is column (x / g) stride +
  // x % g, groups of g contiguous columns stride apart (g = 0: column x)
  int kg, kstride, ng, nstride;
};

__device__ inline int colmap(int x, int g, int stride) { return g ? (x / g) * stride + x % g : x; }

constexpr int kGemmTile = 128;
constexpr int kGemmK = 16;  // K per LDS stage (32 was measured slower: more VGPRs, 36 KB of LDS)

template <bool AT, bool BT, bool MAP>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs g) {
  constexpr int BM = kGemmTile, BN = kGemmTile, BK = kGemmK;
  constexpr int R = BM * BK / 256;  // elements of each operand tile per thread
  // tiles m-major ([row][k]): a lane reads the 4 k values it feeds to the 4
  // MFMAs of a stage with one 16-byte load; a pitch of 20 floats puts the
  // 16 rows of an operand read (and of the stores) on distinct bank groups
  constexpr int LDK = BK + 4;
  static_assert(BK == 16, "one 16-byte read per lane covers the stage's 4 MFMAs");
  __shared__ __attribute__((aligned(16))) float As[BM][LDK];
  __shared__ __attribute__((aligned(16))) float Bs[BN][LDK];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const int kb = blockIdx.z * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  // this thread's 8 elements of the A and B tiles: coalesced along the
  // contiguous dimension of each operand
  int am[R], ak[R], bn[R], bk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (AT) {
      am[r] = t & (BM - 1);
      ak[r] = t / BM + (256 / BM) * r;
    } else {
      ak[r] = t & (BK - 1);
      am[r] = t / BK + (256 / BK) * r;
    }
    if constexpr (BT) {
      bk[r] = t & (BK - 1);
      bn[r] = t / BK + (256 / BK) * r;
    } else {
      bn[r] = t & (BN - 1);
      bk[r] = t / BN + (256 / BN) * r;
    }
  }
  float ra[R], rb[R];
  auto load = [&](int k0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int gm = m0 + am[r], gk = k0 + ak[r];
      ra[r] = (gm < g.M && gk < ke)
                  ? (AT ? g.A[(int64_t)gk * g.lda + gm]
                        : g.A[(int64_t)gm * g.lda + (MAP ? colmap(gk, g.kg, g.kstride) : gk)])
                  : 0.0f;
      const int gn = n0 + bn[r], gk2 = k0 + bk[r];
      rb[r] = (gn < g.N && gk2 < ke) ? (BT ? g.B[(int64_t)gn * g.ldb + gk2] : g.B[(int64_t)gk2 * g.ldb + gn]) : 0.0f;
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += BK) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      As[am[r]][ak[r]] = ra[r];
      Bs[bn[r]][bk[r]] = rb[r];
    }
    __syncthreads();
    if (k0 + BK < ke) load(k0 + BK);
    // MFMA q of the stage takes k = 4 (lane / 16) + q from every lane, for A
    // and B alike: the 4 MFMAs cover the stage's 16 k once each
    f32x4 av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[i] = *(const f32x4*)&As[wm + 16 * i + (lane & 15)][4 * (lane >> 4)];
      bv[i] = *(const f32x4*)&Bs[wn + 16 * i + (lane & 15)][4 * (lane >> 4)];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][q], bv[j][q], acc[i][j], 0, 0, 0);
    __syncthreads();
  }
  // C layout: lane holds rows 4 (lane / 16) + r, column lane % 16 of each 16 x 16 tile
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm + 16 * a + 4 * (lane >> 4) + r;
        const int colm = n0 + wn + 16 * b + (lane & 15);
        if (row < g.M && colm < g.N) {
          float* p = g.Cm + (int64_t)row * g.ldc + (MAP ? colmap(colm, g.ng, g.nstride) : colm);
          if (g.atomic) atomicAdd(p, acc[a][b][r]);
          else *p = acc[a][b][r];
        }
      }
}

// C (+)= A B on v_mfma_f32_16x16x32_bf16 with fp32 accumulation, for
// bf16 inputs: the same operand layouts, tiles (128 x 128, 4 waves of
// 64 x 64), K ranges and store / atomic modes as gemm_f32_kernel, K in
// stages of 32 (stages of 64, at two waves per SIMD, measured 3 % slower
// over the backward).  The operands stay fp32 in memory and are split as they
// are staged into LDS: x = hi + lo with hi = bf16(x) and lo = bf16(x - hi)
// (round to nearest even), about 16 significant bits.  An operand that is
// exact in bf16 (the weight matrices of bf16 inputs) is staged as hi only
// (SA / SB false); the product takes A_hi B_hi + A_lo B_hi + A_hi B_lo
// (the lo lo term is below the fp32 rounding of the sum).  Plain bf16
// operands (hi only on both sides) are not enough here: the position
// gradient cancels to a small fraction of its terms.  An operand tile is
// held in LDS as [row][k] bf16 pairs (k, k + 1) in one dword, 16 pairs per
// row and a pitch of 20 dwords (the 16 rows of a fragment read fall on
// distinct bank groups), so a lane's fragment (8 consecutive k of one row)
// is one 16-byte read.  Each thread stages 8 pairs per operand and stage: with k contiguous in memory (A not transposed, B transposed)
// one 8-byte load per pair, else two 4-byte loads (row-contiguous, so the
// threads' loads of one k are coalesced).  No column maps.
constexpr int kGemmKB = 32;
constexpr int kGemmKP = kGemmKB / 2;     // bf16 pairs per LDS row
constexpr int kGemmPitch = kGemmKP + 4;  // dwords per LDS row
constexpr int kGemmPT = kGemmTile * kGemmKP / 256;  // pairs per thread and operand

template <bool KC>
__device__ inline void bgemm_load(const float* __restrict__ X, int64_t ld, int rows, int row0, int k0, int ke,
                                  f32x2 (&v)[kGemmPT]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int r = 0; r < kGemmPT; ++r) {
    int row, kp;
    if constexpr (KC) {
      kp = t & (kGemmKP - 1);
      row = t / kGemmKP + (256 / kGemmKP) * r;
    } else {
      row = t & 127;
      kp = (t >> 7) + 2 * r;
    }
    const int gr = row0 + row, gk = k0 + 2 * kp;
    f32x2 e = f32x2{0.0f, 0.0f};
    if (gr < rows) {
      if constexpr (KC) {
        const float* p = X + (int64_t)gr * ld + gk;
        if (gk + 1 < ke) e = *(const f32x2*)p;
        else if (gk < ke) e.x = p[0];
      } else {
        if (gk < ke) e.x = X[(int64_t)gk * ld + gr];
        if (gk + 1 < ke) e.y = X[(int64_t)(gk + 1) * ld + gr];
      }
    }
    v[r] = e;
  }
}

template <bool KC, bool SPLIT>
__device__ inline void bgemm_store(uint32_t (*Sh)[kGemmPitch], uint32_t (*Sl)[kGemmPitch],
                                   const f32x2 (&v)[kGemmPT]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int r = 0; r < kGemmPT; ++r) {
    const int row = KC ? t / kGemmKP + (256 / kGemmKP) * r : t & 127;
    const int kp = KC ? t & (kGemmKP - 1) : (t >> 7) + 2 * r;
    const bf16x2 hi = __builtin_convertvector(v[r], bf16x2);
    Sh[row][kp] = __builtin_bit_cast(uint32_t, hi);
    if constexpr (SPLIT) {
      const f32x2 rest = v[r] - __builtin_convertvector(hi, f32x2);
      Sl[row][kp] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2));
    }
  }
}

__device__ inline f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

template <bool AT, bool BT, bool SA, bool SB>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(GemmArgs g) {
  constexpr int BM = kGemmTile, BN = kGemmTile, BK = kGemmKB;
  __shared__ __attribute__((aligned(16))) uint32_t Ah[BM][kGemmPitch];
  __shared__ __attribute__((aligned(16))) uint32_t Al[SA ? BM : 1][kGemmPitch];
  __shared__ __attribute__((aligned(16))) uint32_t Bh[BN][kGemmPitch];
  __shared__ __attribute__((aligned(16))) uint32_t Bl[SB ? BN : 1][kGemmPitch];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const int kb = blockIdx.z * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  // A(m, k): k contiguous unless AT; B(k, n) = B[n ldb + k]: k contiguous when BT
  f32x2 ra[kGemmPT], rb[kGemmPT];
  auto load = [&](int k0) {
    bgemm_load<!AT>(g.A, g.lda, g.M, m0, k0, ke, ra);
    bgemm_load<BT>(g.B, g.ldb, g.N, n0, k0, ke, rb);
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += BK) {
    bgemm_store<!AT, SA>(Ah, Al, ra);
    bgemm_store<BT, SB>(Bh, Bl, rb);
    __syncthreads();
    if (k0 + BK < ke) load(k0 + BK);
    // fragments of MFMA K step h: row lane % 16 of the tile, k = 32 h + 8
    // (lane / 16) .. + 7
#pragma unroll
    for (int h = 0; h < kGemmKB / 32; ++h) {
      const int fo = 16 * h + 4 * (lane >> 4);
      u32x4 ah[4], al[4], bh[4], bl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ri = wm + 16 * i + (lane & 15), rj = wn + 16 * i + (lane & 15);
        ah[i] = *(const u32x4*)&Ah[ri][fo];
        bh[i] = *(const u32x4*)&Bh[rj][fo];
        if constexpr (SA) al[i] = *(const u32x4*)&Al[ri][fo];
        if constexpr (SB) bl[i] = *(const u32x4*)&Bl[rj][fo];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = mfma_bf16(ah[i], bh[j], acc[i][j]);
          if constexpr (SA) acc[i][j] = mfma_bf16(al[i], bh[j], acc[i][j]);
          if constexpr (SB) acc[i][j] = mfma_bf16(ah[i], bl[j], acc[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm + 16 * a + 4 * (lane >> 4) + r;
        const int colm = n0 + wn + 16 * b + (lane & 15);
        if (row < g.M && colm < g.N) {
          float* p = g.Cm + (int64_t)row * g.ldc + colm;
          if (g.atomic) atomicAdd(p, acc[a][b][r]);
          else *p = acc[a][b][r];
        }
      }
}

// How the bf16-operand GEMM stages its operands: not at all (the fp32
// GEMM runs), or A split into hi + lo with B exact in bf16, or both split.
enum GemmSplit { kSplitNone = 0, kSplitA = 1, kSplitAB = 2 };

// fp32 GEMM, or with split != kSplitNone the bf16-operand GEMM above (no
// column maps; the k-contiguous operands need 8-byte aligned rows, else the
// fp32 kernel runs)
template <bool AT, bool BT>
so2_status gemm(const float* A, int64_t lda, const float* B, int64_t ldb, float* Cm, int64_t ldc, int M, int N, int K,
                bool atomic, hipStream_t stream, int kg = 0, int kstride = 0, int ng = 0, int nstride = 0,
                GemmSplit split = kSplitNone) {
  if (M <= 0 || N <= 0 || K <= 0) return SO2_OK;
  GemmArgs g{A, B, Cm, M, N, K, lda, ldb, ldc, K, atomic ? 1 : 0, kg, kstride, ng, nstride};
  const bool aligned = (AT || (lda % 2 == 0 && ((uintptr_t)A & 7) == 0)) &&
                       (!BT || (ldb % 2 == 0 && ((uintptr_t)B & 7) == 0));
  if (split != kSplitNone && !kg && !ng && aligned) {
    unsigned splits = 1;
    if (atomic) {
      const int64_t tiles = (int64_t)((M + kGemmTile - 1) / kGemmTile) * ((N + kGemmTile - 1) / kGemmTile);
      const int64_t want = std::max<int64_t>(1, 2048 / std::max<int64_t>(tiles, 1));
      const int64_t by_k = std::max<int64_t>(1, K / 512);
      splits = (unsigned)std::min(want, by_k);
      g.k_split = (int)(((K + splits - 1) / splits + kGemmKB - 1) / kGemmKB * kGemmKB);
      splits = (unsigned)((K + g.k_split - 1) / g.k_split);
    }
    const dim3 grid((unsigned)((M + kGemmTile - 1) / kGemmTile), (unsigned)((N + kGemmTile - 1) / kGemmTile), splits);
    if (split == kSplitA) hipLaunchKernelGGL((gemm_bf16_kernel<AT, BT, true, false>), grid, dim3(256), 0, stream, g);
    else hipLaunchKernelGGL((gemm_bf16_kernel<AT, BT, true, true>), grid, dim3(256), 0, stream, g);
    SO2_CHECK_LAUNCH();
    return SO2_OK;
  }
  unsigned splits = 1;
  if (atomic) {
    // K ranges of at least 512 so that the tile grid covers the device
    const int64_t tiles = (int64_t)((M + kGemmTile - 1) / kGemmTile) * ((N + kGemmTile - 1) / kGemmTile);
    const int64_t want = std::max<int64_t>(1, 2048 / std::max<int64_t>(tiles, 1));
    const int64_t by_k = std::max<int64_t>(1, K / 512);
    splits = (unsigned)std::min(want, by_k);
    g.k_split = (int)(((K + splits - 1) / splits + kGemmK - 1) / kGemmK * kGemmK);
    splits = (unsigned)((K + g.k_split - 1) / g.k_split);
  }
  if (kg || ng)
    hipLaunchKernelGGL((gemm_f32_kernel<AT, BT, true>),
                       dim3((unsigned)((M + kGemmTile - 1) / kGemmTile), (unsigned)((N + kGemmTile - 1) / kGemmTile),
                            splits),
                       dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<AT, BT, false>),
                       dim3((unsigned)((M + kGemmTile - 1) / kGemmTile), (unsigned)((N + kGemmTile - 1) / kGemmTile),
                            splits),
                       dim3(256), 0, stream, g);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

// ---------------------------------------------------------------- weights

// B_m in fp32 from w_so2: W0 for m = 0, [[W1, -W2], [W2, W1]] for m >= 1,
// for the blocks m <= m_max.  With F focus streams, w_so2 is F stacks of
// C' = C / F channels (each W0 and (W1_m, W2_m) for m = 1..m_max), and B_m
// is stored as F dense stream matrices: stream f's rows and columns are the
// block's (group, c') with c' < C', a group being one (sign, l) of the block
// (l for m = 0), i.e. the block's columns group * C + f C' + c'.
template <typename T>
__global__ void __launch_bounds__(256) bmat_build_kernel(const T* __restrict__ w, float* __restrict__ bm, int L, int C,
                                                         int m_max, int F) {
  const int m = blockIdx.y;
  const int wd = blk_width(L, C, m) / F;  // one stream matrix is wd x wd
  const int64_t per = (int64_t)wd * wd;
  const int64_t n = per * F;
  const int cf = C / F;
  const int64_t stack = so2_w1_offset(L, cf, m_max + 1);  // entries of one stream's stack
  float* out = bm + bmat_off(L, C, m, F);
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x) {
    const int f = (int)(q / per);
    const int o = (int)((q % per) / wd), in = (int)(q % wd);
    const int go = o / cf, co = o % cf, gi = in / cf, ci = in % cf;
    float v;
    if (m == 0) {
      const int64_t k0 = (int64_t)(L + 1) * cf;
      v = load_as_float(w + f * stack, ((int64_t)go * cf + co) * k0 + (int64_t)gi * cf + ci);
    } else {
      const int kg = L + 1 - m;  // groups per sign
      const int so = go / kg, si = gi / kg;
      const int64_t kmf = (int64_t)kg * cf;
      const T* w1 = w + f * stack + so2_w1_offset(L, cf, m);
      const T* w2 = w1 + kmf * kmf;
      const int64_t r = ((int64_t)(go % kg) * cf + co) * kmf + (int64_t)(gi % kg) * cf + ci;
      v = so == si ? load_as_float(w1, r) : (so == 0 ? -load_as_float(w2, r) : load_as_float(w2, r));
    }
    out[q] = v;
  }
}

// dW from dB: dW0 = dB_0; dW1 = dB_m[+,+] + dB_m[-,-]; dW2 = dB_m[-,+] - dB_m[+,-].
__global__ void __launch_bounds__(256) dw_fold_kernel(const float* __restrict__ db, float* __restrict__ dw, int L,
                                                      int C) {
  const int m = blockIdx.y;
  const int wd = blk_width(L, C, m);
  const float* src = db + bmat_off(L, C, m);
  if (m == 0) {
    const int64_t n = (int64_t)wd * wd;
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x)
      dw[q] = src[q];
    return;
  }
  const int km = wd / 2;
  const int64_t n = (int64_t)km * km;
  float* d1 = dw + so2_w1_offset(L, C, m);
  float* d2 = d1 + n;
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x) {
    const int ro = (int)(q / km), ri = (int)(q % km);
    const float pp = src[(int64_t)ro * wd + ri], mm = src[(int64_t)(km + ro) * wd + km + ri];
    const float mp = src[(int64_t)(km + ro) * wd + ri], pm = src[(int64_t)ro * wd + km + ri];
    d1[q] = pp + mm;
    d2[q] = mp - pm;
  }
}

// dst[i] = src[i] in fp32 (W_q and W_k for the projection GEMMs).
template <typename T>
__global__ void __launch_bounds__(256) to_f32_kernel(const void* src, float* __restrict__ dst, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = load_as_float((const T*)src, i);
}

// dw[c][o] += sum over a block of atoms of x[a][0][c] g[a][o] (g = dq or dk)
constexpr int kProjAtoms = 256;
template <typename T>
__global__ void __launch_bounds__(256) proj_bwd_dw_kernel(const void* x, const float* __restrict__ g, float* dw,
                                                          int n_rows, int nc, int C) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)C * C) return;
  const int c = (int)(idx / C), o = (int)(idx % C);
  const int a0 = blockIdx.y * kProjAtoms, a1 = min(a0 + kProjAtoms, n_rows);
  float acc = 0.0f;
  for (int a = a0; a < a1; ++a) acc += load_as_float((const T*)x, (int64_t)a * nc * C + c) * g[(int64_t)a * C + o];
  atomicAdd(dw + idx, acc);
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

// The rotation generators J_a (wigner_generators' recursion, one degree at a
// time): wave a takes axis a, its lanes the entries of each degree, which
// depend on degree l - 1 of the same axis and on the identity.
__global__ void __launch_bounds__(192) generators_kernel(float* gen, int L) {
  constexpr int kTot = wig_total(kMaxL);
  __shared__ float ident[kTot];
  __shared__ float J[3][kTot];
  const int t = threadIdx.x, ax = t / 64, lane = t % 64;
  const int tot = wig_total(L);
  for (int q = t; q < tot; q += 192) ident[q] = 0.0f;
  __syncthreads();
  for (int l = 0; l <= L; ++l)
    for (int m = t; m < 2 * l + 1; m += 192) ident[wig_offset(l) + m * (2 * l + 1) + m] = 1.0f;
  if (lane == 0) {
    J[ax][0] = 0.0f;
    if (L >= 1) {
      // [e_a]x for a = x, y, z, row-major
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
      wigner_l1(E, &J[ax][wig_offset(1)]);
    }
  }
  __syncthreads();
  for (int l = 2; l <= L; ++l) {
    const int n = 2 * l + 1;
    const float* J1 = &J[ax][wig_offset(1)];
    const float* Jp = &J[ax][wig_offset(l - 1)];
    const float* I1 = ident + wig_offset(1);
    const float* Ip = ident + wig_offset(l - 1);
    for (int q = lane; q < n * n; q += 64)
      J[ax][wig_offset(l) + q] =
          wigner_entry(l, q / n - l, q % n - l, J1, Ip) + wigner_entry(l, q / n - l, q % n - l, I1, Jp);
    __syncthreads();
  }
  for (int q = lane; q < tot; q += 64) gen[ax * tot + q] = J[ax][q];
}

so2_status fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (!p || n <= 0) return SO2_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

// ---------------------------------------------------------------- workspace

// Edges per batch: 64 per target, between 4096 and 65536.
int64_t batch_edges(int n_targets) {
  const int64_t want = ((int64_t)n_targets * 64 + 255) / 256 * 256;
  return std::min<int64_t>(65536, std::max<int64_t>(4096, want));
}

size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

// Offsets (bytes) of the backward's scratch arrays.
struct BwdScratch {
  size_t dq, dk, gen, wq, wk, smax, sinv, sbar, bm, db, xt, yt, D, g, gp, dg, phi, a, ab, sc, tgt, total;
  int64_t cap;
  BwdScratch(int n_atoms, int n_targets, int L, int C, int H, int K) {
    cap = batch_edges(n_targets);
    const size_t nc = (size_t)n_comp(L), nw = (size_t)wig_total(L);
    const size_t nb = (size_t)bmat_off(L, C, L + 1);
    size_t o = 0;
    auto take = [&](size_t bytes) {
      const size_t at = o;
      o += al256(bytes);
      return at;
    };
    dq = take(4 * (size_t)n_targets * C);
    dk = take(4 * (size_t)n_atoms * C);
    gen = take(4 * 3 * nw);
    wq = take(4 * (size_t)C * C);
    wk = take(4 * (size_t)C * C);
    smax = take(4 * (size_t)n_targets * H);
    sinv = take(4 * (size_t)n_targets * H);
    sbar = take(4 * (size_t)n_targets * H);
    bm = take(4 * nb);
    db = take(4 * nb);
    xt = take(4 * (size_t)cap * nc * C);
    yt = take(4 * (size_t)cap * nc * C);
    D = take(4 * (size_t)cap * nw);
    g = take(4 * (size_t)cap * C);
    gp = take(4 * (size_t)cap * C);
    dg = take(4 * (size_t)cap * C);
    phi = take(4 * (size_t)cap * K);
    a = take(4 * (size_t)cap * H);
    ab = take(4 * (size_t)cap * H);
    sc = take(4 * (size_t)cap * kScal);
    tgt = take(4 * (size_t)cap);
    total = o;
  }
};

template <int L, typename T>
so2_status launch_edges(int which, const BatchParams& P, hipStream_t stream) {
  const unsigned grid = (unsigned)std::min<int64_t>(P.nb, kGridCap);
  if (grid == 0) return SO2_OK;
  switch (which) {
    case 0:
      hipLaunchKernelGGL(batch_targets_kernel, dim3((unsigned)((P.nb + 255) / 256)), dim3(256), 0, stream, P);
      SO2_CHECK_LAUNCH();
      hipLaunchKernelGGL((bwd_prep_kernel<L, T>), dim3(grid), dim3(kLane), 0, stream, P);
      break;
    case 1: hipLaunchKernelGGL((bwd_sbar_kernel<L>), dim3(grid), dim3(kLane), 0, stream, P); break;
    case 2: hipLaunchKernelGGL((bwd_dyt_kernel<L>), dim3(grid), dim3(kLane), 0, stream, P); break;
    case 3: hipLaunchKernelGGL((bwd_final_kernel<L, T>), dim3(grid), dim3(kLane), 0, stream, P); break;
    case 4: hipLaunchKernelGGL((fwd_finish_kernel<L, T>), dim3(grid), dim3(kLane), 0, stream, P); break;
    default: hipLaunchKernelGGL((fwd_target_kernel<L, T>), dim3(grid), dim3(kTargetThreads), 0, stream, P); break;
  }
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

template <typename T>
so2_status edges_dispatch(int L, int which, const BatchParams& P, hipStream_t stream) {
  switch (L) {
    case 0: return launch_edges<0, T>(which, P, stream);
    case 1: return launch_edges<1, T>(which, P, stream);
    case 2: return launch_edges<2, T>(which, P, stream);
    case 3: return launch_edges<3, T>(which, P, stream);
    case 4: return launch_edges<4, T>(which, P, stream);
    case 5: return launch_edges<5, T>(which, P, stream);
    default: return launch_edges<6, T>(which, P, stream);
  }
}

so2_status run_edges(int L, int dtype, int which, const BatchParams& P, hipStream_t stream) {
  return dtype == SO2_BF16 ? edges_dispatch<uint16_t>(L, which, P, stream) : edges_dispatch<float>(L, which, P, stream);
}

so2_status run_stats(int dtype, const BatchParams& P, hipStream_t stream) {
  const unsigned grid = (unsigned)std::min(P.n_targets, kGridCap);
  if (grid == 0) return SO2_OK;
  if (dtype == SO2_BF16) hipLaunchKernelGGL(batch_stats_kernel<uint16_t>, dim3(grid), dim3(kLane), 0, stream, P);
  else hipLaunchKernelGGL(batch_stats_kernel<float>, dim3(grid), dim3(kLane), 0, stream, P);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

// Edge range [row_ptr[0], row_ptr[n_targets]) read back to the host: the
// batch plan needs it (one wait on the stream).
so2_status edge_range(const int32_t* row_ptr, int n_targets, int64_t* first, int64_t* count, hipStream_t stream) {
  int32_t ends[2] = {0, 0};
  if (n_targets > 0) {
    SO2_CHECK(hipMemcpyAsync(&ends[0], row_ptr, sizeof(int32_t), hipMemcpyDeviceToHost, stream));
    SO2_CHECK(hipMemcpyAsync(&ends[1], row_ptr + n_targets, sizeof(int32_t), hipMemcpyDeviceToHost, stream));
    SO2_CHECK(hipStreamSynchronize(stream));
  }
  *first = ends[0];
  *count = (int64_t)ends[1] - ends[0];
  return *count < 0 ? SO2_ERR_INVALID_ARGUMENT : SO2_OK;
}

// Offsets (bytes) of the forward's scratch arrays.
struct FwdScratch {
  size_t smax, sinv, bm, xt, yt, D, a, ab, tgt, total;
  int64_t cap;
  FwdScratch(int n_targets, int L, int C, int H, int m_max, int F) {
    cap = batch_edges(n_targets);
    const size_t nc = (size_t)n_comp(L), nw = (size_t)wig_total(L);
    const size_t nb = (size_t)bmat_off(L, C, m_max + 1, F);
    size_t o = 0;
    auto take = [&](size_t bytes) {
      const size_t at = o;
      o += al256(bytes);
      return at;
    };
    smax = take(4 * (size_t)n_targets * H);
    sinv = take(4 * (size_t)n_targets * H);
    bm = take(4 * nb);
    xt = take(4 * (size_t)cap * nc * C);
    yt = take(4 * (size_t)cap * nc * C);
    D = take(4 * (size_t)cap * nw);
    a = take(4 * (size_t)cap * H);
    ab = take(4 * (size_t)cap * H);
    tgt = take(4 * (size_t)cap);
    total = o;
  }
};

}  // namespace

bool bwd_supported(int L, int C, int H, int K) {
  return L >= 0 && L <= kMaxL && C >= 1 && C <= 256 && H >= 1 && H <= kMaxHeadsB && C % H == 0 && K >= 2;
}

size_t bwd_scratch_bytes(int n_atoms, int n_targets, int L, int C, int H, int K) {
  return BwdScratch(n_atoms, n_targets, L, C, H, K).total;
}

bool batch_fwd_supported(int L, int C, int H, int K, int m_max, int n_focus) {
  return bwd_supported(L, C, H, K) && m_max >= 0 && m_max <= L && n_focus >= 1 && n_focus <= kMaxHeadsB &&
         C % n_focus == 0;
}

size_t batch_fwd_scratch_bytes(int n_targets, int L, int C, int H, int m_max, int n_focus) {
  return FwdScratch(n_targets, L, C, H, m_max, n_focus).total;
}

so2_status launch_attention_batch_fwd(const AttnArgs& a, hipStream_t stream) {
  const int L = a.L, C = a.C, nc = n_comp(L), mm = a.m_max;
  const FwdScratch S(a.n_targets, L, C, a.H, mm, a.n_focus);
  char* ws = (char*)a.scratch;
  so2_status st;
  if ((st = fill_zero(a.y, (int64_t)a.n_targets * nc * C, stream)) != SO2_OK) return st;
  int64_t e_first = 0, n_edges = 0;
  if ((st = edge_range(a.row_ptr, a.n_targets, &e_first, &n_edges, stream)) != SO2_OK) return st;
  if (n_edges == 0) return SO2_OK;

  float* bm = (float*)(ws + S.bm);
  if (a.dtype == SO2_BF16)
    hipLaunchKernelGGL(bmat_build_kernel<uint16_t>, dim3(1024, mm + 1), dim3(256), 0, stream,
                       (const uint16_t*)a.w_so2, bm, L, C, mm, a.n_focus);
  else
    hipLaunchKernelGGL(bmat_build_kernel<float>, dim3(1024, mm + 1), dim3(256), 0, stream, (const float*)a.w_so2, bm,
                       L, C, mm, a.n_focus);
  SO2_CHECK_LAUNCH();

  BatchParams P{};
  P.pos = a.pos;
  P.y = a.y;
  P.w_logit = a.w_logit;
  P.w_focus = a.w_focus;
  P.m_max = mm;
  P.n_focus = a.n_focus;
  P.row_ptr = a.row_ptr;
  P.col = a.col;
  P.x = a.x;
  P.w_rad = a.w_rad;
  P.q = a.q;
  P.k = a.k;
  P.smax = (float*)(ws + S.smax);
  P.sinv = (float*)(ws + S.sinv);
  P.b.xt = (float*)(ws + S.xt);
  P.b.yt = (float*)(ws + S.yt);
  P.b.D = (float*)(ws + S.D);
  P.b.a = (float*)(ws + S.a);
  P.b.ab = (float*)(ws + S.ab);
  P.b.tgt = (int32_t*)(ws + S.tgt);
  P.n_targets = a.n_targets;
  P.C = C;
  P.H = a.H;
  P.K = a.K;
  P.p = a.p;
  P.cutoff = a.cutoff;
  P.flags = a.flags;
  P.periodic = a.periodic;
  for (int d = 0; d < 3; ++d) P.box[d] = a.box[d];
  if ((st = run_stats(a.dtype, P, stream)) != SO2_OK) return st;

  const int64_t cap = S.cap;
  const int64_t ld = (int64_t)nc * C;
  for (int64_t b = 0; b * cap < n_edges; ++b) {
    P.e0 = e_first + b * cap;
    P.nb = (int32_t)std::min<int64_t>(cap, n_edges - b * cap);
    if ((st = run_edges(L, a.dtype, 0, P, stream)) != SO2_OK) return st;
    // per stream f: Y_m[:, f cols] = X_m[:, f cols] B_m,f^T, the stream's
    // columns taken as groups of C' (one per (sign, l)) C apart
    const int F = a.n_focus, cf = C / F;
    for (int m = 0; m <= mm; ++m) {
      const int wd = blk_width(L, C, m) / F;
      const int64_t xo = blk_off(L, C, m);
      for (int f = 0; f < F; ++f) {
        const float* bf = bm + bmat_off(L, C, m, F) + (int64_t)f * wd * wd;
        st = F == 1 ? gemm<false, true>(P.b.xt + xo, ld, bf, wd, P.b.yt + xo, ld, P.nb, wd, wd, false, stream)
                    : gemm<false, true>(P.b.xt + xo + f * cf, ld, bf, wd, P.b.yt + xo + f * cf, ld, P.nb, wd, wd, false,
                                        stream, cf, C, cf, C);
        if (st != SO2_OK) return st;
      }
    }
    if (C <= kTargetThreads) {
      // one workgroup per target: the messages stay in registers
      if ((st = run_edges(L, a.dtype, 5, P, stream)) != SO2_OK) return st;
    } else {
      if ((st = run_edges(L, a.dtype, 4, P, stream)) != SO2_OK) return st;
      const unsigned rgrid = (unsigned)std::min<int64_t>(P.nb, kGridCap);
      hipLaunchKernelGGL(fwd_reduce_kernel, dim3(rgrid), dim3(256), 0, stream, P, (int)ld);
      SO2_CHECK_LAUNCH();
    }
  }
  return SO2_OK;
}

so2_status launch_attention_bwd(const AttnArgs& a, const float* dy, float* dx, float* dpos, float* dw_q, float* dw_k,
                                float* dw_rad, float* dw_so2, hipStream_t stream) {
  const int L = a.L, C = a.C;
  const int nc = n_comp(L);
  const BwdScratch S(a.n_atoms, a.n_targets, L, a.C, a.H, a.K);
  char* ws = (char*)a.scratch;
  float* dq = (float*)(ws + S.dq);
  float* dk = (float*)(ws + S.dk);
  float* gen = (float*)(ws + S.gen);
  float* smax = (float*)(ws + S.smax);
  float* sinv = (float*)(ws + S.sinv);
  float* sbar = (float*)(ws + S.sbar);
  float* bm = (float*)(ws + S.bm);
  float* db = (float*)(ws + S.db);
  const bool radial = !(a.flags & SO2_FLAG_NO_RADIAL);
  so2_status st;
  if ((st = fill_zero(dx, (int64_t)a.n_atoms * nc * C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dpos, (int64_t)a.n_atoms * 3, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dq, (int64_t)a.n_targets * C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dk, (int64_t)a.n_atoms * C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(sbar, (int64_t)a.n_targets * a.H, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dw_q, (int64_t)C * C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dw_k, (int64_t)C * C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dw_rad, (int64_t)a.K * C, stream)) != SO2_OK) return st;
  if (dw_so2 && (st = fill_zero(db, bmat_off(L, C, L + 1), stream)) != SO2_OK) return st;

  int64_t e_first = 0, n_edges = 0;
  if ((st = edge_range(a.row_ptr, a.n_targets, &e_first, &n_edges, stream)) != SO2_OK) return st;

  if (n_edges > 0) {
    hipLaunchKernelGGL(generators_kernel, dim3(1), dim3(192), 0, stream, gen, L);
    SO2_CHECK_LAUNCH();
    const unsigned nbw = 1024;
    if (a.dtype == SO2_BF16)
      hipLaunchKernelGGL(bmat_build_kernel<uint16_t>, dim3(nbw, L + 1), dim3(256), 0, stream,
                         (const uint16_t*)a.w_so2, bm, L, C, L, 1);
    else
      hipLaunchKernelGGL(bmat_build_kernel<float>, dim3(nbw, L + 1), dim3(256), 0, stream, (const float*)a.w_so2,
                         bm, L, C, L, 1);
    SO2_CHECK_LAUNCH();

    BatchParams P{};
    P.pos = a.pos;
    P.row_ptr = a.row_ptr;
    P.col = a.col;
    P.x = a.x;
    P.w_rad = a.w_rad;
    P.m_max = L;
    P.n_focus = 1;
    P.dy = dy;
    P.q = a.q;
    P.k = a.k;
    P.gen = gen;
    P.smax = smax;
    P.sinv = sinv;
    P.sbar = sbar;
    P.dq = dq;
    P.dk = dk;
    P.dx = dx;
    P.dpos = dpos;
    P.b.xt = (float*)(ws + S.xt);
    P.b.yt = (float*)(ws + S.yt);
    P.b.D = (float*)(ws + S.D);
    P.b.g = (float*)(ws + S.g);
    P.b.gp = (float*)(ws + S.gp);
    P.b.dg = (float*)(ws + S.dg);
    P.b.phi = (float*)(ws + S.phi);
    P.b.a = (float*)(ws + S.a);
    P.b.ab = (float*)(ws + S.ab);
    P.b.sc = (float*)(ws + S.sc);
    P.b.tgt = (int32_t*)(ws + S.tgt);
    P.n_targets = a.n_targets;
    P.C = C;
    P.H = a.H;
    P.K = a.K;
    P.p = a.p;
    P.cutoff = a.cutoff;
    P.flags = a.flags;
    P.periodic = a.periodic;
    for (int d = 0; d < 3; ++d) P.box[d] = a.box[d];

    if ((st = run_stats(a.dtype, P, stream)) != SO2_OK) return st;

    const int64_t cap = S.cap;
    const int64_t nbat = (n_edges + cap - 1) / cap;
    const int64_t ld = (int64_t)nc * C;
    // bf16 inputs: the per-m maps on the matrix cores' bf16 path, each fp32
    // operand split into two bf16 parts (the weight matrices are exact in
    // bf16); fp32 inputs: fp32 GEMMs
    const bool bf16 = a.dtype == SO2_BF16;
    const GemmSplit sp_a = bf16 ? kSplitA : kSplitNone, sp_ab = bf16 ? kSplitAB : kSplitNone;
    auto set_batch = [&](int64_t b) {
      P.e0 = e_first + b * cap;
      P.nb = (int32_t)std::min<int64_t>(cap, n_edges - b * cap);
    };
    // forward map of the batch: Y_m = X_m B_m^T
    auto forward_map = [&]() -> so2_status {
      for (int m = 0; m <= L; ++m) {
        const int wd = blk_width(L, C, m);
        const int64_t xo = blk_off(L, C, m);
        so2_status s2 = gemm<false, true>(P.b.xt + xo, ld, bm + bmat_off(L, C, m), wd, P.b.yt + xo, ld, P.nb, wd, wd,
                                          false, stream, 0, 0, 0, 0, sp_a);
        if (s2 != SO2_OK) return s2;
      }
      return SO2_OK;
    };
    // pass 1: Sbar
    for (int64_t b = 0; b < nbat; ++b) {
      set_batch(b);
      if ((st = run_edges(L, a.dtype, 0, P, stream)) != SO2_OK) return st;
      if ((st = forward_map()) != SO2_OK) return st;
      if ((st = run_edges(L, a.dtype, 1, P, stream)) != SO2_OK) return st;
    }
    // pass 2: gradients, the batch still in the buffers first
    for (int64_t bb = nbat - 1; bb >= 0; --bb) {
      set_batch(bb);
      if (bb != nbat - 1) {
        if ((st = run_edges(L, a.dtype, 0, P, stream)) != SO2_OK) return st;
        if ((st = forward_map()) != SO2_OK) return st;
      }
      if ((st = run_edges(L, a.dtype, 2, P, stream)) != SO2_OK) return st;
      for (int m = 0; m <= L; ++m) {
        const int wd = blk_width(L, C, m);
        const int64_t xo = blk_off(L, C, m);
        // dB_m += dY_m^T X_m (before dX overwrites X)
        if (dw_so2 &&
            (st = gemm<true, false>(P.b.yt + xo, ld, P.b.xt + xo, ld, db + bmat_off(L, C, m), wd, wd, wd, P.nb, true,
                                    stream, 0, 0, 0, 0, sp_ab)) != SO2_OK)
          return st;
        // dX_m = dY_m B_m, over X_m
        if ((st = gemm<false, false>(P.b.yt + xo, ld, bm + bmat_off(L, C, m), wd, P.b.xt + xo, ld, P.nb, wd, wd, false,
                                     stream, 0, 0, 0, 0, sp_a)) != SO2_OK)
          return st;
      }
      if ((st = run_edges(L, a.dtype, 3, P, stream)) != SO2_OK) return st;
      // dW_rad += phi^T dg
      if (dw_rad && radial &&
          (st = gemm<true, false>(P.b.phi, a.K, P.b.dg, C, dw_rad, C, a.K, C, P.nb, true, stream)) != SO2_OK)
        return st;
    }
    if (dw_so2) {
      hipLaunchKernelGGL(dw_fold_kernel, dim3(1024, L + 1), dim3(256), 0, stream, db, dw_so2, L, C);
      SO2_CHECK_LAUNCH();
    }
  } else if (dw_so2) {
    if ((st = fill_zero(dw_so2, so2_w1_offset(L, C, L + 1), stream)) != SO2_OK) return st;
  }

  // the projections of the l = 0 slice: dx[., 0, .] += dq W_q^T + dk W_k^T
  // as fp32 GEMMs (weights widened once)
  float* wq32 = (float*)(ws + S.wq);
  float* wk32 = (float*)(ws + S.wk);
  const int64_t cc = (int64_t)C * C;
  const unsigned gcc = (unsigned)std::min<int64_t>((cc + 255) / 256, 1024);
  if (a.dtype == SO2_BF16) {
    hipLaunchKernelGGL(to_f32_kernel<uint16_t>, dim3(gcc), dim3(256), 0, stream, a.w_q, wq32, cc);
    hipLaunchKernelGGL(to_f32_kernel<uint16_t>, dim3(gcc), dim3(256), 0, stream, a.w_k, wk32, cc);
  } else {
    hipLaunchKernelGGL(to_f32_kernel<float>, dim3(gcc), dim3(256), 0, stream, a.w_q, wq32, cc);
    hipLaunchKernelGGL(to_f32_kernel<float>, dim3(gcc), dim3(256), 0, stream, a.w_k, wk32, cc);
  }
  SO2_CHECK_LAUNCH();
  const int64_t ldx = (int64_t)nc * C;
  if ((st = gemm<false, true>(dq, C, wq32, C, dx, ldx, a.n_targets, C, C, true, stream)) != SO2_OK) return st;
  if ((st = gemm<false, true>(dk, C, wk32, C, dx, ldx, a.n_atoms, C, C, true, stream)) != SO2_OK) return st;
  const unsigned gw = (unsigned)((cc + 255) / 256);
  if (dw_q && a.n_targets > 0) {
    if (a.dtype == SO2_BF16)
      hipLaunchKernelGGL(proj_bwd_dw_kernel<uint16_t>, dim3(gw, (a.n_targets + kProjAtoms - 1) / kProjAtoms),
                         dim3(256), 0, stream, a.x, dq, dw_q, a.n_targets, nc, C);
    else
      hipLaunchKernelGGL(proj_bwd_dw_kernel<float>, dim3(gw, (a.n_targets + kProjAtoms - 1) / kProjAtoms), dim3(256),
                         0, stream, a.x, dq, dw_q, a.n_targets, nc, C);
    SO2_CHECK_LAUNCH();
  }
  if (dw_k && a.n_atoms > 0) {
    if (a.dtype == SO2_BF16)
      hipLaunchKernelGGL(proj_bwd_dw_kernel<uint16_t>, dim3(gw, (a.n_atoms + kProjAtoms - 1) / kProjAtoms),
                         dim3(256), 0, stream, a.x, dk, dw_k, a.n_atoms, nc, C);
    else
      hipLaunchKernelGGL(proj_bwd_dw_kernel<float>, dim3(gw, (a.n_atoms + kProjAtoms - 1) / kProjAtoms), dim3(256),
                         0, stream, a.x, dk, dw_k, a.n_atoms, nc, C);
    SO2_CHECK_LAUNCH();
  }
  return SO2_OK;
}

}  // namespace so2
