// General fused SO(2) attention forward, fp32 arithmetic on the vector ALUs.
//
// Any L <= 6, C <= 256, fp32 or bf16 inputs.  This is the fp32 path (the
// precision the tiny configuration is checked at) and the path for shapes
// the bf16 MFMA kernel does not cover.  One workgroup (256 lanes) per target
// atom; nothing per edge leaves the workgroup.
//
// Method ("E2Former-V2: On-the-Fly Equivariant Attention with Linear
// Activation Memory", technical summary, sections 2.1 and 2.2; envelope
// from "EquiformerV3: Scaling Efficient, Expressive, and General SE(3)-Equivariant
// Graph Attention Transformers", technical summary, section 2.B.3):
//   sweep 1 (online softmax statistics): for each head a running maximum
//     of the logits and a running normaliser sum_j u_ij exp(z_ij - max),
//     rescaled whenever the maximum grows; lanes combine their partial
//     (max, sum) pairs at the end.
//   sweep 2, per neighbour j in order:
//     geometry r_ij = mic(p_j - p_i), envelope u, edge frame R, Wigner-D
//     blocks D^l(R) (recursion, parallel over entries), radial gate g[c],
//     final weight w^h = u exp(z^h - max^h) / sum^h;
//     xt = g * D x_j; yt = per-m map of xt; acc += w^{h(c)} D^T yt.
//   Because the weights of sweep 2 are already normalised, the accumulator
//   is never rescaled.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "wigner.h"

namespace so2 {

constexpr int kValuThreads = 256;

struct ValuParams {
  const float* pos;
  const int32_t* row_ptr;
  const int32_t* col;
  const void* x;
  const void* w_rad;
  const void* w_so2;
  const float* q;
  const float* k;
  float* y;
  int32_t L, C, H, K, p;
  float cutoff;
  uint32_t flags;
  int32_t periodic;
  float box[3];
  int32_t m_max, n_focus;
  const void* w_logit;  // [K][H] or null
  const void* w_focus;  // [C] when n_focus > 1
};

// Radial logit bias of head h: sum_k phi_k(rho) w_logit[k][h] (0 without it).
template <typename T>
__device__ inline float logit_bias(const ValuParams& P, float rho, int h) {
  if (!P.w_logit) return 0.0f;
  const float step = P.cutoff / (float)(P.K - 1);
  const float inv2s2 = 1.0f / (2.0f * step * step);
  float b = 0.0f;
  for (int kk = 0; kk < P.K; ++kk) {
    const float dr = rho - step * (float)kk;
    b += expf(-dr * dr * inv2s2) * load_as_float((const T*)P.w_logit, (int64_t)kk * P.H + h);
  }
  return b;
}

__device__ inline float block_reduce_max(float v, float* red) {
  int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = kValuThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  float r = red[0];
  __syncthreads();
  return r;
}

__device__ inline float block_reduce_sum(float v, float* red) {
  int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = kValuThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  float r = red[0];
  __syncthreads();
  return r;
}

template <typename T>
__global__ void __launch_bounds__(kValuThreads) attn_valu_kernel(ValuParams P) {
  const int i = blockIdx.x;
  const int t = threadIdx.x;
  const int L = P.L, C = P.C, H = P.H;
  const int nc = n_comp(L);
  const int d = C / H;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  const int nwig = (wig_total(L) + 3) & ~3;

  extern __shared__ float smem[];
  float* s_xt = smem;           // [nc][C] rotated, gated input
  float* s_yt = s_xt + nc * C;  // [nc][C] after the per-m map
  float* s_acc = s_yt + nc * C; // [nc][C] accumulator
  float* s_D = s_acc + nc * C;  // Wigner-D blocks
  float* s_g = s_D + nwig;      // [C] radial gate
  float* s_q = s_g + C;         // [C] q_i
  float* s_w = s_q + C;         // [H] weights of the current edge
  float* s_M = s_w + H;         // [H] softmax max
  float* s_S = s_M + H;         // [H] 1 / normaliser
  float* s_geo = s_S + H;       // [16] r, rho, u, R
  float* s_red = s_geo + 16;    // [kValuThreads]

  const T* x = (const T*)P.x;
  const T* w_rad = (const T*)P.w_rad;
  const T* w_so2 = (const T*)P.w_so2;
  const int e0 = P.row_ptr[i], e1 = P.row_ptr[i + 1];
  const float rc = P.cutoff;

  for (int c = t; c < C; c += kValuThreads) s_q[c] = P.q[(int64_t)i * C + c];
  for (int a = t; a < nc * C; a += kValuThreads) s_acc[a] = 0.0f;
  __syncthreads();

  // ---- sweep 1: online softmax statistics, one head at a time
  for (int h = 0; h < H; ++h) {
    float m = -INFINITY, s = 0.0f;
    for (int e = e0 + t; e < e1; e += kValuThreads) {
      int j = P.col[e];
      const EdgeGeo geo = edge_geometry(P.pos, i, j, P.periodic, P.box, rc);
      float u = envelope_u(geo.s, geo.t, P.p);
      float z = 0.0f;
      for (int c = h * d; c < (h + 1) * d; ++c) z += s_q[c] * P.k[(int64_t)j * C + c];
      z = z * inv_sqrt_d + logit_bias<T>(P, geo.rho, h);
      if (z > m) {
        s = s * expf(m - z) + u;
        m = z;
      } else {
        s += u * expf(z - m);
      }
    }
    float M = block_reduce_max(m, s_red);
    float part = (m == -INFINITY) ? 0.0f : s * expf(m - M);
    float S = block_reduce_sum(part, s_red);
    if (t == 0) {
      s_M[h] = M;
      s_S[h] = S > 0.0f ? 1.0f / S : 0.0f;
    }
  }
  __syncthreads();

  // ---- sweep 2: values
  for (int e = e0; e < e1; ++e) {
    const int j = P.col[e];
    if (t == 0) {
      const EdgeGeo geo = edge_geometry(P.pos, i, j, P.periodic, P.box, rc);
      const float rho = geo.rho;
      float inv = rho > 0.0f ? 1.0f / rho : 0.0f;
      s_geo[0] = rho;
      s_geo[1] = envelope_u(geo.s, geo.t, P.p);
      edge_frame(geo.r[0] * inv, geo.r[1] * inv, geo.r[2] * inv, s_geo + 4);
    }
    __syncthreads();
    // Wigner-D: degree 0 and 1 directly, then one degree at a time.
    if (t == 0) s_D[0] = 1.0f;
    if (L >= 1 && t < 9) {
      const int ax[3] = {1, 2, 0};
      int a = t / 3, b = t % 3;
      s_D[wig_offset(1) + t] = s_geo[4 + ax[a] * 3 + ax[b]];
    }
    __syncthreads();
    for (int l = 2; l <= L; ++l) {
      const int n = 2 * l + 1;
      for (int q = t; q < n * n; q += kValuThreads)
        s_D[wig_offset(l) + q] =
            wigner_entry(l, q / n - l, q % n - l, s_D + wig_offset(1), s_D + wig_offset(l - 1));
      __syncthreads();
    }
    const float rho = s_geo[0];
    const float u = s_geo[1];
    // radial gate and attention weights of this edge
    for (int c = t; c < C; c += kValuThreads) {
      float g = 1.0f;
      if (!(P.flags & SO2_FLAG_NO_RADIAL)) {
        const float mu_step = rc / (float)(P.K - 1);
        const float inv2s2 = 1.0f / (2.0f * mu_step * mu_step);
        g = 0.0f;
        for (int kk = 0; kk < P.K; ++kk) {
          float dr = rho - mu_step * (float)kk;
          g += expf(-dr * dr * inv2s2) * load_as_float(w_rad, (int64_t)kk * C + c);
        }
        if (P.flags & SO2_FLAG_RBF_ENVELOPE) g *= u;
      }
      s_g[c] = g;
    }
    for (int h = t; h < H; h += kValuThreads) {
      float z = 0.0f;
      for (int c = h * d; c < (h + 1) * d; ++c) z += s_q[c] * P.k[(int64_t)j * C + c];
      z = z * inv_sqrt_d + logit_bias<T>(P, rho, h);
      s_w[h] = u * expf(z - s_M[h]) * s_S[h];
    }
    __syncthreads();
    // rotate into the edge frame and gate: xt[(l,m),c] = g[c] sum_m' D^l[m][m'] x_j[(l,m'),c]
    const T* xj = x + (int64_t)j * nc * C;
    for (int a = t; a < nc * C; a += kValuThreads) {
      int comp = a / C, c = a % C;
      int l = (int)sqrtf((float)comp + 0.5f);
      int mrow = comp - l * l;  // m + l
      const float* Dl = s_D + wig_offset(l) + mrow * (2 * l + 1);
      float v = 0.0f;
      for (int b = 0; b < 2 * l + 1; ++b) v += Dl[b] * load_as_float(xj, (int64_t)(l * l + b) * C + c);
      s_xt[a] = v * s_g[c];
    }
    __syncthreads();
    // per-m map: one output row per wave lane group, lanes split the inputs.
    // With F focus streams, stream f = cp / Cf owns its stack of maps over
    // its Cf channels (stack f at f * so2_w1_offset(L, Cf, m_max + 1));
    // orders above m_max give 0.
    {
      const int lane = t & 63;
      const int wave = t >> 6;
      const int Cf = C / P.n_focus;
      const int64_t stack = so2_w1_offset(L, Cf, P.m_max + 1);
      for (int o = wave; o < nc * C; o += kValuThreads / 64) {
        int comp = o / C, cp = o % C;
        int l = (int)sqrtf((float)comp + 0.5f);
        int m = comp - l * l - l;
        int am = m < 0 ? -m : m;
        const int f = cp / Cf, cpf = cp - f * Cf;
        const T* ws = w_so2 + f * stack;
        float acc = 0.0f;
        if (am > P.m_max) {
        } else if (am == 0) {
          const int64_t K0 = (int64_t)(L + 1) * Cf;
          const T* row = ws + ((int64_t)l * Cf + cpf) * K0;
          for (int kk = lane; kk < K0; kk += 64) {
            int lp = kk / Cf, c = f * Cf + kk % Cf;
            acc += load_as_float(row, kk) * s_xt[(lp * lp + lp) * C + c];
          }
        } else {
          const int64_t Km = (int64_t)(L + 1 - am) * Cf;
          const int64_t off1 = so2_w1_offset(L, Cf, am);
          const T* row1 = ws + off1 + ((int64_t)(l - am) * Cf + cpf) * Km;
          const T* row2 = row1 + Km * Km;
          for (int kk = lane; kk < Km; kk += 64) {
            int lp = kk / Cf + am, c = f * Cf + kk % Cf;
            float xp = s_xt[(lp * lp + lp + am) * C + c];
            float xm = s_xt[(lp * lp + lp - am) * C + c];
            float w1 = load_as_float(row1, kk), w2 = load_as_float(row2, kk);
            acc += (m > 0) ? (w1 * xp - w2 * xm) : (w2 * xp + w1 * xm);
          }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (lane == 0) s_yt[o] = acc;
      }
    }
    __syncthreads();
    // cross-focus softmax: pi_f from the streams' invariant l = 0 message,
    // score_f = sum_{c in f} w_focus[c] yt[(0,0), c]; stream f scaled by pi_f
    if (P.n_focus > 1) {
      const int F = P.n_focus, Cf = C / F;
      if (t == 0) {
        float mx = -INFINITY;
        for (int f = 0; f < F; ++f) {
          float sc = 0.0f;
          for (int c = f * Cf; c < (f + 1) * Cf; ++c) sc += load_as_float((const T*)P.w_focus, c) * s_yt[c];
          s_red[f] = sc;
          mx = fmaxf(mx, sc);
        }
        float sum = 0.0f;
        for (int f = 0; f < F; ++f) {
          s_red[f] = expf(s_red[f] - mx);
          sum += s_red[f];
        }
        for (int f = 0; f < F; ++f) s_red[f] /= sum;
      }
      __syncthreads();
      for (int a = t; a < nc * C; a += kValuThreads) s_yt[a] *= s_red[(a % C) / Cf];
      __syncthreads();
    }
    // rotate back and accumulate: acc[(l,m'),c] += w^{h(c)} sum_m D^l[m][m'] yt[(l,m),c]
    for (int a = t; a < nc * C; a += kValuThreads) {
      int comp = a / C, c = a % C;
      int l = (int)sqrtf((float)comp + 0.5f);
      int mcol = comp - l * l;
      const int n = 2 * l + 1;
      const float* Dl = s_D + wig_offset(l);
      float v = 0.0f;
      for (int b = 0; b < n; ++b) v += Dl[b * n + mcol] * s_yt[(l * l + b) * C + c];
      s_acc[a] += s_w[c / d] * v;
    }
    __syncthreads();
  }

  float* yi = P.y + (int64_t)i * nc * C;
  for (int a = t; a < nc * C; a += kValuThreads) yi[a] = s_acc[a];
}

bool valu_supported(int L, int C, int H) {
  return L >= 0 && L <= kMaxL && C >= 1 && C <= 256 && H >= 1 && C % H == 0 && H <= C;
}

size_t valu_scratch_bytes(int, int) { return 0; }

static size_t valu_smem_bytes(int L, int C, int H) {
  const int nc = n_comp(L);
  const int nwig = (wig_total(L) + 3) & ~3;
  return sizeof(float) * (size_t)(3 * nc * C + nwig + 2 * C + 3 * H + 16 + kValuThreads);
}

so2_status launch_attention_valu(const AttnArgs& a, hipStream_t stream) {
  ValuParams P{};
  P.pos = a.pos;
  P.row_ptr = a.row_ptr;
  P.col = a.col;
  P.x = a.x;
  P.w_rad = a.w_rad;
  P.w_so2 = a.w_so2;
  P.q = a.q;
  P.k = a.k;
  P.y = a.y;
  P.L = a.L;
  P.C = a.C;
  P.H = a.H;
  P.K = a.K;
  P.p = a.p;
  P.cutoff = a.cutoff;
  P.flags = a.flags;
  P.periodic = a.periodic;
  for (int d = 0; d < 3; ++d) P.box[d] = a.box[d];
  P.m_max = a.m_max;
  P.n_focus = a.n_focus;
  P.w_logit = a.w_logit;
  P.w_focus = a.w_focus;
  const size_t smem = valu_smem_bytes(a.L, a.C, a.H);
  if (a.n_targets == 0) return SO2_OK;
  if (a.dtype == SO2_BF16) {
    SO2_CHECK(hipFuncSetAttribute((const void*)attn_valu_kernel<uint16_t>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem));
    hipLaunchKernelGGL(attn_valu_kernel<uint16_t>, dim3(a.n_targets), dim3(kValuThreads), smem,
                       stream, P);
  } else {
    SO2_CHECK(hipFuncSetAttribute((const void*)attn_valu_kernel<float>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem));
    hipLaunchKernelGGL(attn_valu_kernel<float>, dim3(a.n_targets), dim3(kValuThreads), smem,
                       stream, P);
  }
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

}  // namespace so2
