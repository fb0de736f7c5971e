// Backward of the fused SO(2) attention forward, fp32 on the vector ALUs.
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
// Nothing per edge is stored: like the forward, one workgroup per target
// recomputes every edge (rotation, gate, per-m map, rotation back), and
// only the softmax statistics per (target, head) are kept between sweeps:
//   sweep 0   running max M and normaliser sum_j u_ij exp(z_ij - M);
//   sweep 1   per edge v_ij and s_ij^h = <dy_i, v_ij> over the channels of
//             head h; Sbar^h = sum_j a_ij^h s_ij^h;
//   sweep 2   per edge, again v_ij and s_ij^h, then
//     dL/dz^h = a^h (s^h - Sbar^h),  dL/du = sum_h abar^h (s^h - Sbar^h)
//     (abar = a / u = exp(z - M) / normaliser),
//     dv = a (.) dy_i,  dyt = D dv,  dW_so2 += per-m outer products of dyt
//     and xt,  dxt = W^T dyt (the transposed per-m map),
//     dg[c] = sum_(l,m) dxt xh (xh = D x_j before the gate),
//     dx_j += D^T (dxt (.) g),  dW_rad += phi dg,
//     d|r| = sum_c dg[c] dg_c/d|r| + dL/du du/d|r|,
//     direction: a rotation w of the edge direction r_hat -> r_hat + w x
//     r_hat is a frame R exp(-[w]x), so D -> D (I - sum_a w_a J_a) with J_a
//     the rotation generators in the real harmonic basis, and
//       dL/dw_a = <dv, J_a v> - <dxt (.) g, D J_a x_j>;
//     the direction gradient is (dL/dw) x r_hat, so
//       dL/dr = (dL/dw) x r_hat / |r| + d|r| r_hat,
//     added to dpos[j] and taken from dpos[i];
//     dq_i += dz k_j / sqrt(d), dk_j += dz q_i / sqrt(d).
// A second kernel takes dq and dk through the projections of the l = 0
// slice: dx[.,0,.] += dq W_q^T + dk W_k^T, dW_q = x0^T dq, dW_k = x0^T dk.
// Gradients that several workgroups add to (dx of sources, dpos, dk and the
// weights) use fp32 atomics, so their summation order varies between runs.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "wigner.h"

namespace so2 {

namespace {

constexpr int kBwdThreads = 256;

struct BwdParams {
  const float* pos;
  const int32_t* row_ptr;
  const int32_t* col;
  const void* x;
  const void* w_q;
  const void* w_k;
  const void* w_rad;
  const void* w_so2;
  const float* dy;
  const float* q;    // [n_atoms][C]
  const float* k;    // [n_atoms][C]
  const float* gen;  // [3][wig_total(L)] rotation generators
  float* dq;         // [n_targets][C]
  float* dk;         // [n_atoms][C]
  float* dx;
  float* dpos;
  float* dw_rad;  // or null
  float* dw_so2;  // or null
  int32_t n_atoms, n_targets, L, C, H, K, p;
  float cutoff;
  uint32_t flags;
  int32_t periodic;
  float box[3];
};

// LDS layout of the backward kernel, in floats.
struct BwdLds {
  int nc, C, H, K, nwig;
  int G, XH, XT, Y, V, D, DJ, J, g, gp, dg, q, dq, phi, dwr, M, S, a, ab, s, sbar, red, total;
  __host__ __device__ BwdLds(int L, int C_, int H_, int K_) : nc((L + 1) * (L + 1)), C(C_), H(H_), K(K_) {
    nwig = (wig_total(L) + 3) & ~3;
    int o = 0;
    G = o;  // dy_i
    o += nc * C;
    XH = o;  // D x_j
    o += nc * C;
    XT = o;  // gated
    o += nc * C;
    Y = o;  // yt, then dyt
    o += nc * C;
    V = o;  // v, then dxt
    o += nc * C;
    D = o;
    o += nwig;
    DJ = o;  // D J_a
    o += 3 * nwig;
    J = o;  // generators
    o += 3 * nwig;
    g = o;
    o += C;
    gp = o;  // dg/d|r|
    o += C;
    dg = o;
    o += C;
    q = o;
    o += C;
    dq = o;
    o += C;
    phi = o;  // phi_k (times u with the envelope flag)
    o += (K + 3) & ~3;
    dwr = o;  // dW_rad of this target
    o += K * C;
    M = o;
    o += H;
    S = o;  // 1 / normaliser
    o += H;
    a = o;
    o += H;
    ab = o;
    o += H;
    s = o;
    o += H;
    sbar = o;
    o += H;
    red = o;  // scalars: [0] d|r| (radial part), [1..3] dir1, [4..6] dir2, [8..] geometry
    o += 32;
    total = o;
  }
};

__device__ inline void atomic_add_f(float* p, float v) { atomicAdd(p, v); }

// Sum v over the wave and add it to *dst from lane 0 (LDS atomics).
__device__ inline void wave_add(float* dst, float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) atomicAdd(dst, v);
}

template <typename T>
__global__ void __launch_bounds__(kBwdThreads) attn_bwd_kernel(BwdParams P) {
  const int i = blockIdx.x;
  const int t = threadIdx.x;
  const int L = P.L, C = P.C, H = P.H, K = P.K;
  const int nc = n_comp(L);
  const int d = C / H;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  const int e0 = P.row_ptr[i], e1 = P.row_ptr[i + 1];
  float* dqo = P.dq + (int64_t)i * C;
  if (e0 == e1) {
    for (int c = t; c < C; c += kBwdThreads) dqo[c] = 0.0f;
    return;
  }
  extern __shared__ float sm[];
  const BwdLds Ly(L, C, H, K);
  float* sG = sm + Ly.G;
  float* sXH = sm + Ly.XH;
  float* sXT = sm + Ly.XT;
  float* sY = sm + Ly.Y;
  float* sV = sm + Ly.V;
  float* sD = sm + Ly.D;
  float* sDJ = sm + Ly.DJ;
  float* sJ = sm + Ly.J;
  float* sg = sm + Ly.g;
  float* sgp = sm + Ly.gp;
  float* sdg = sm + Ly.dg;
  float* sq = sm + Ly.q;
  float* sdq = sm + Ly.dq;
  float* sphi = sm + Ly.phi;
  float* sdwr = sm + Ly.dwr;
  float* sM = sm + Ly.M;
  float* sS = sm + Ly.S;
  float* sa = sm + Ly.a;
  float* sab = sm + Ly.ab;
  float* ss = sm + Ly.s;
  float* ssb = sm + Ly.sbar;
  float* sred = sm + Ly.red;
  const int nw = wig_total(L);
  const float rc = P.cutoff;
  const bool radial = !(P.flags & SO2_FLAG_NO_RADIAL);
  const bool rbf_env = (P.flags & SO2_FLAG_RBF_ENVELOPE) != 0;
  const float mu_step = rc / (float)(K - 1);
  const float inv2s2 = 1.0f / (2.0f * mu_step * mu_step);

  for (int a = t; a < nc * C; a += kBwdThreads) sG[a] = P.dy[(int64_t)i * nc * C + a];
  for (int a = t; a < 3 * nw; a += kBwdThreads) sJ[(a / nw) * Ly.nwig + a % nw] = P.gen[a];
  for (int c = t; c < C; c += kBwdThreads) {
    sq[c] = P.q[(int64_t)i * C + c];
    sdq[c] = 0.0f;
  }
  for (int a = t; a < K * C; a += kBwdThreads) sdwr[a] = 0.0f;
  for (int h = t; h < H; h += kBwdThreads) ssb[h] = 0.0f;

  // ---- sweep 0: softmax statistics (per head, online over the edges)
  for (int h = t; h < H; h += kBwdThreads) {
    float m = -INFINITY, sum = 0.0f;
    for (int e = e0; e < e1; ++e) {
      const int j = P.col[e];
      const EdgeGeo geo = edge_geometry(P.pos, i, j, P.periodic, P.box, rc);
      const float u = envelope_u(geo.s, geo.t, P.p);
      float z = 0.0f;
      for (int c = h * d; c < (h + 1) * d; ++c) z += P.q[(int64_t)i * C + c] * P.k[(int64_t)j * C + c];
      z *= inv_sqrt_d;
      if (z > m) {
        sum = sum * expf(m - z) + u;
        m = z;
      } else {
        sum += u * expf(z - m);
      }
    }
    sM[h] = m;
    sS[h] = sum > 0.0f ? 1.0f / sum : 0.0f;
  }
  __syncthreads();
  bool degenerate = false;
  for (int h = 0; h < H; ++h) degenerate |= !(sS[h] > 0.0f);
  if (degenerate) {  // every envelope is 0: the layer output is 0 and not differentiable
    for (int c = t; c < C; c += kBwdThreads) dqo[c] = 0.0f;
    return;
  }

  const T* w_so2 = (const T*)P.w_so2;
  for (int sweep = 1; sweep <= 2; ++sweep) {
    for (int e = e0; e < e1; ++e) {
      const int j = P.col[e];
      // geometry, frame, envelope, softmax weights of the edge
      if (t == 0) {
        const EdgeGeo geo = edge_geometry(P.pos, i, j, P.periodic, P.box, rc);
        const float inv = geo.rho > 0.0f ? 1.0f / geo.rho : 0.0f;
        sred[8] = geo.rho;
        sred[9] = envelope_u(geo.s, geo.t, P.p);
        sred[10] = envelope_du(geo.s, geo.t, P.p) / rc;  // du/d|r|
        sred[11] = geo.r[0] * inv;
        sred[12] = geo.r[1] * inv;
        sred[13] = geo.r[2] * inv;
        edge_frame(sred[11], sred[12], sred[13], sred + 16);
        for (int q = 0; q < 7; ++q) sred[q] = 0.0f;
      }
      for (int h = t; h < H; h += kBwdThreads) ss[h] = 0.0f;
      __syncthreads();
      const float rho = sred[8], u = sred[9], dudr = sred[10];
      // Wigner-D: degree 0 and 1 directly, then one degree at a time
      if (t == 0) sD[0] = 1.0f;
      if (L >= 1 && t < 9) {
        const int ax[3] = {1, 2, 0};
        sD[wig_offset(1) + t] = sred[16 + ax[t / 3] * 3 + ax[t % 3]];
      }
      if (t < K) {
        const float dr = rho - mu_step * (float)t;
        const float ph = expf(-dr * dr * inv2s2);
        sphi[t] = rbf_env ? ph * u : ph;
      }
      for (int h = t; h < H; h += kBwdThreads) {
        float z = 0.0f;
        for (int c = h * d; c < (h + 1) * d; ++c) z += sq[c] * P.k[(int64_t)j * C + c];
        z *= inv_sqrt_d;
        const float ab = expf(z - sM[h]) * sS[h];
        sab[h] = ab;
        sa[h] = u * ab;
      }
      __syncthreads();
      for (int l = 2; l <= L; ++l) {
        const int n = 2 * l + 1;
        for (int q = t; q < n * n; q += kBwdThreads)
          sD[wig_offset(l) + q] = wigner_entry(l, q / n - l, q % n - l, sD + wig_offset(1), sD + wig_offset(l - 1));
        __syncthreads();
      }
      // radial gate and its derivative along |r|
      for (int c = t; c < C; c += kBwdThreads) {
        float g = 1.0f, gp = 0.0f;
        if (radial) {
          g = 0.0f;
          float g0 = 0.0f;  // sum_k phi_k W (no envelope factor)
          for (int kk = 0; kk < K; ++kk) {
            const float dr = rho - mu_step * (float)kk;
            const float ph = expf(-dr * dr * inv2s2);
            const float w = load_as_float((const T*)P.w_rad, (int64_t)kk * C + c);
            g0 += ph * w;
            gp += -dr * 2.0f * inv2s2 * ph * w;
          }
          g = rbf_env ? g0 * u : g0;
          if (rbf_env) gp = gp * u + g0 * dudr;
        }
        sg[c] = g;
        sgp[c] = gp;
      }
      // D J_a (per degree) for the direction gradient
      if (sweep == 2) {
        for (int q = t; q < 3 * nw; q += kBwdThreads) {
          const int ax = q / nw, r = q % nw;
          int l = 0;
          while (wig_offset(l + 1) <= r) ++l;
          const int n = 2 * l + 1, o = r - wig_offset(l), m = o / n, mp = o % n;
          const float* Dl = sD + wig_offset(l) + m * n;
          const float* Jl = sJ + ax * Ly.nwig + wig_offset(l);
          float acc = 0.0f;
          for (int b = 0; b < n; ++b) acc += Dl[b] * Jl[b * n + mp];
          sDJ[ax * Ly.nwig + r] = acc;
        }
      }
      __syncthreads();
      // xh = D x_j, xt = g xh
      const T* xj = (const T*)P.x + (int64_t)j * nc * C;
      for (int a = t; a < nc * C; a += kBwdThreads) {
        const int comp = a / C, c = a % C;
        const int l = (int)sqrtf((float)comp + 0.5f);
        const float* Dl = sD + wig_offset(l) + (comp - l * l) * (2 * l + 1);
        float v = 0.0f;
        for (int b = 0; b < 2 * l + 1; ++b) v += Dl[b] * load_as_float(xj, (int64_t)(l * l + b) * C + c);
        sXH[a] = v;
        sXT[a] = v * sg[c];
      }
      __syncthreads();
      // yt = per-m map of xt: one output row per wave, lanes split the inputs
      {
        const int lane = t & 63, wave = t >> 6;
        for (int o = wave; o < nc * C; o += kBwdThreads / 64) {
          const int comp = o / C, cp = o % C;
          const int l = (int)sqrtf((float)comp + 0.5f);
          const int m = comp - l * l - l, am = m < 0 ? -m : m;
          float acc = 0.0f;
          if (am == 0) {
            const int64_t K0 = (int64_t)(L + 1) * C;
            const T* row = w_so2 + ((int64_t)l * C + cp) * K0;
            for (int kk = lane; kk < K0; kk += 64) {
              const int lp = kk / C, c = kk % C;
              acc += load_as_float(row, kk) * sXT[(lp * lp + lp) * C + c];
            }
          } else {
            const int64_t Km = (int64_t)(L + 1 - am) * C;
            const T* row1 = w_so2 + so2_w1_offset(L, C, am) + ((int64_t)(l - am) * C + cp) * Km;
            const T* row2 = row1 + Km * Km;
            for (int kk = lane; kk < Km; kk += 64) {
              const int lp = kk / C + am, c = kk % C;
              const float xp = sXT[(lp * lp + lp + am) * C + c], xm = sXT[(lp * lp + lp - am) * C + c];
              const float w1 = load_as_float(row1, kk), w2 = load_as_float(row2, kk);
              acc += m > 0 ? (w1 * xp - w2 * xm) : (w2 * xp + w1 * xm);
            }
          }
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
          if (lane == 0) sY[o] = acc;
        }
      }
      __syncthreads();
      // v = D^T yt; s^h = <dy_i, v> over the head's channels
      for (int a = t; a < nc * C; a += kBwdThreads) {
        const int comp = a / C, c = a % C;
        const int l = (int)sqrtf((float)comp + 0.5f);
        const int n = 2 * l + 1, mcol = comp - l * l;
        const float* Dl = sD + wig_offset(l);
        float v = 0.0f;
        for (int b = 0; b < n; ++b) v += Dl[b * n + mcol] * sY[(l * l + b) * C + c];
        sV[a] = v;
        atomicAdd(&ss[c / d], sG[a] * v);
      }
      __syncthreads();
      if (sweep == 1) {
        for (int h = t; h < H; h += kBwdThreads) ssb[h] += sa[h] * ss[h];
        __syncthreads();
        continue;
      }
      // ---- sweep 2: gradients of this edge
      // dir1_a = <dv, J_a v> with dv = a (.) dy_i
      for (int a = t; a < ((nc * C + 63) & ~63); a += kBwdThreads) {
        float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f;
        if (a < nc * C) {
          const int comp = a / C, c = a % C;
          const int l = (int)sqrtf((float)comp + 0.5f);
          const int n = 2 * l + 1, m = comp - l * l;
          const float dv = sa[c / d] * sG[a];
          const float* J0 = sJ + wig_offset(l) + m * n;
          for (int b = 0; b < n; ++b) {
            const float vb = sV[(l * l + b) * C + c];
            p0 += J0[b] * vb;
            p1 += J0[Ly.nwig + b] * vb;
            p2 += J0[2 * Ly.nwig + b] * vb;
          }
          p0 *= dv;
          p1 *= dv;
          p2 *= dv;
        }
        wave_add(sred + 1, p0);
        wave_add(sred + 2, p1);
        wave_add(sred + 3, p2);
      }
      // dyt = D dv (into sY)
      for (int a = t; a < nc * C; a += kBwdThreads) {
        const int comp = a / C, c = a % C;
        const int l = (int)sqrtf((float)comp + 0.5f);
        const int n = 2 * l + 1;
        const float* Dl = sD + wig_offset(l) + (comp - l * l) * n;
        float v = 0.0f;
        for (int b = 0; b < n; ++b) v += Dl[b] * sG[(l * l + b) * C + c];
        sY[a] = v * sa[c / d];
      }
      __syncthreads();
      // dW_so2 += per-m outer products (dyt, xt)
      if (P.dw_so2) {
        const int64_t k0 = (int64_t)(L + 1) * C;
        for (int64_t q = t; q < k0 * k0; q += kBwdThreads) {
          const int64_t r = q / k0, cc = q % k0;
          const int l = (int)(r / C), lp = (int)(cc / C);
          const float gv = sY[(l * l + l) * C + r % C] * sXT[(lp * lp + lp) * C + cc % C];
          if (gv != 0.0f) atomic_add_f(P.dw_so2 + q, gv);
        }
        for (int m = 1; m <= L; ++m) {
          const int64_t km = (int64_t)(L + 1 - m) * C;
          float* d1 = P.dw_so2 + so2_w1_offset(L, C, m);
          float* d2 = d1 + km * km;
          for (int64_t q = t; q < km * km; q += kBwdThreads) {
            const int64_t r = q / km, cc = q % km;
            const int l = (int)(r / C) + m, lp = (int)(cc / C) + m;
            const float yp = sY[(l * l + l + m) * C + r % C], ym = sY[(l * l + l - m) * C + r % C];
            const float xp = sXT[(lp * lp + lp + m) * C + cc % C], xm = sXT[(lp * lp + lp - m) * C + cc % C];
            atomic_add_f(d1 + q, yp * xp + ym * xm);
            atomic_add_f(d2 + q, ym * xp - yp * xm);
          }
        }
      }
      // dxt = W^T dyt (transposed per-m map), one output per lane: the lanes
      // of a wave read consecutive columns of a weight row
      for (int a = t; a < nc * C; a += kBwdThreads) {
        const int comp = a / C, c = a % C;
        const int lp = (int)sqrtf((float)comp + 0.5f);
        const int m = comp - lp * lp - lp, am = m < 0 ? -m : m;
        float acc = 0.0f;
        if (am == 0) {
          const int64_t K0 = (int64_t)(L + 1) * C;
          const int64_t col = (int64_t)lp * C + c;
          for (int l = 0; l <= L; ++l)
            for (int cp = 0; cp < C; ++cp)
              acc += load_as_float(w_so2, ((int64_t)l * C + cp) * K0 + col) * sY[(l * l + l) * C + cp];
        } else {
          const int64_t Km = (int64_t)(L + 1 - am) * C;
          const T* w1 = w_so2 + so2_w1_offset(L, C, am);
          const T* w2 = w1 + Km * Km;
          const int64_t col = (int64_t)(lp - am) * C + c;
          for (int l = am; l <= L; ++l)
            for (int cp = 0; cp < C; ++cp) {
              const int64_t r = ((int64_t)(l - am) * C + cp) * Km + col;
              const float yp = sY[(l * l + l + am) * C + cp], ym = sY[(l * l + l - am) * C + cp];
              const float a1 = load_as_float(w1, r), a2 = load_as_float(w2, r);
              // xt_+ grad: W1^T dy_+ + W2^T dy_- ; xt_- grad: -W2^T dy_+ + W1^T dy_-
              acc += m > 0 ? (a1 * yp + a2 * ym) : (a1 * ym - a2 * yp);
            }
        }
        sV[a] = acc;
      }
      __syncthreads();
      // dg[c], d|r| (radial), dir2_a = <dxt g, D J_a x_j>, dx_j += D^T (dxt g)
      for (int c = t; c < C; c += kBwdThreads) {
        float dg = 0.0f;
        for (int comp = 0; comp < nc; ++comp) dg += sV[comp * C + c] * sXH[comp * C + c];
        sdg[c] = dg;
      }
      float* dxj = P.dx + (int64_t)j * nc * C;
      for (int a = t; a < ((nc * C + 63) & ~63); a += kBwdThreads) {
        float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f;
        if (a < nc * C) {
          const int comp = a / C, c = a % C;
          const int l = (int)sqrtf((float)comp + 0.5f);
          const int n = 2 * l + 1, mrow = comp - l * l;
          const float gx = sV[a] * sg[c];
          const float* R0 = sDJ + wig_offset(l) + mrow * n;
          for (int b = 0; b < n; ++b) {
            const float xb = load_as_float(xj, (int64_t)(l * l + b) * C + c);
            p0 += R0[b] * xb;
            p1 += R0[Ly.nwig + b] * xb;
            p2 += R0[2 * Ly.nwig + b] * xb;
          }
          p0 *= gx;
          p1 *= gx;
          p2 *= gx;
          // dx_j[(l, b), c] += sum_m D[m][b] dxt[(l, m), c] g[c]: column b = mrow here
          const float* Dl = sD + wig_offset(l);
          float dxv = 0.0f;
          for (int mm = 0; mm < n; ++mm) dxv += Dl[mm * n + mrow] * sV[(l * l + mm) * C + c];
          atomic_add_f(dxj + a, dxv * sg[c]);
        }
        wave_add(sred + 4, p0);
        wave_add(sred + 5, p1);
        wave_add(sred + 6, p2);
      }
      __syncthreads();
      // radial parts, softmax parts, W_rad, q/k
      for (int c = t; c < ((C + 63) & ~63); c += kBwdThreads) wave_add(sred + 0, c < C ? sdg[c] * sgp[c] : 0.0f);
      if (radial)
        for (int a = t; a < K * C; a += kBwdThreads) sdwr[a] += sphi[a / C] * sdg[a % C];
      for (int c = t; c < C; c += kBwdThreads) {
        const int h = c / d;
        const float dz = sa[h] * (ss[h] - ssb[h]) * inv_sqrt_d;
        sdq[c] += dz * P.k[(int64_t)j * C + c];
        atomic_add_f(P.dk + (int64_t)j * C + c, dz * sq[c]);
      }
      __syncthreads();
      if (t == 0) {
        float du = 0.0f;
        for (int h = 0; h < H; ++h) du += sab[h] * (ss[h] - ssb[h]);
        const float drho = sred[0] + du * dudr;
        const float w0 = sred[1] - sred[4], w1 = sred[2] - sred[5], w2 = sred[3] - sred[6];
        const float rx = sred[11], ry = sred[12], rz = sred[13];
        const float inv = rho > 0.0f ? 1.0f / rho : 0.0f;
        // (dL/dw) x r_hat / |r| + d|r| r_hat
        const float gx = (w1 * rz - w2 * ry) * inv + drho * rx;
        const float gy = (w2 * rx - w0 * rz) * inv + drho * ry;
        const float gz = (w0 * ry - w1 * rx) * inv + drho * rz;
        atomic_add_f(P.dpos + 3 * (int64_t)j + 0, gx);
        atomic_add_f(P.dpos + 3 * (int64_t)j + 1, gy);
        atomic_add_f(P.dpos + 3 * (int64_t)j + 2, gz);
        atomic_add_f(P.dpos + 3 * (int64_t)i + 0, -gx);
        atomic_add_f(P.dpos + 3 * (int64_t)i + 1, -gy);
        atomic_add_f(P.dpos + 3 * (int64_t)i + 2, -gz);
      }
      __syncthreads();
    }
    __syncthreads();
  }
  for (int c = t; c < C; c += kBwdThreads) dqo[c] = sdq[c];
  if (P.dw_rad && radial)
    for (int a = t; a < K * C; a += kBwdThreads) atomic_add_f(P.dw_rad + a, sdwr[a]);
}

// dx[a][0][c] += sum_o dq[a][o] w_q[c][o] (a < n_targets) + sum_o dk[a][o] w_k[c][o]
template <typename T>
__global__ void __launch_bounds__(256) proj_bwd_dx_kernel(const float* __restrict__ dq, const float* __restrict__ dk,
                                                          const void* w_q, const void* w_k, float* __restrict__ dx,
                                                          int n_atoms, int n_targets, int nc, int C) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_atoms * C) return;
  const int a = (int)(idx / C), c = (int)(idx % C);
  float acc = 0.0f;
  if (a < n_targets)
    for (int o = 0; o < C; ++o) acc += dq[(int64_t)a * C + o] * load_as_float((const T*)w_q, (int64_t)c * C + o);
  for (int o = 0; o < C; ++o) acc += dk[(int64_t)a * C + o] * load_as_float((const T*)w_k, (int64_t)c * C + o);
  dx[(int64_t)a * nc * C + c] += acc;
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

__global__ void generators_kernel(float* gen, float* scratch, int L) {
  if (threadIdx.x == 0 && blockIdx.x == 0) wigner_generators(L, gen, scratch);
}

so2_status fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (!p || n <= 0) return SO2_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

}  // namespace

bool bwd_supported(int L, int C, int H, int K) {
  if (!(L >= 0 && L <= kMaxL && C >= 1 && H >= 1 && C % H == 0 && K >= 2)) return false;
  const BwdLds Ly(L, C, H, K);
  return sizeof(float) * (size_t)Ly.total <= 160 * 1024;
}

size_t bwd_scratch_bytes(int n_atoms, int n_targets, int L, int C) {
  const size_t a = (sizeof(float) * (size_t)n_targets * C + 255) & ~(size_t)255;  // dq
  const size_t b = (sizeof(float) * (size_t)n_atoms * C + 255) & ~(size_t)255;    // dk
  const size_t g = (sizeof(float) * 6 * (size_t)wig_total(L) + 255) & ~(size_t)255;  // generators + scratch
  return a + b + g;
}

so2_status launch_attention_bwd(const AttnArgs& a, const float* dy, float* dx, float* dpos, float* dw_q, float* dw_k,
                                float* dw_rad, float* dw_so2, hipStream_t stream) {
  const int nc = n_comp(a.L);
  char* ws = (char*)a.scratch;
  float* dq = (float*)ws;
  float* dk = (float*)(ws + ((sizeof(float) * (size_t)a.n_targets * a.C + 255) & ~(size_t)255));
  float* gen = (float*)((char*)dk + ((sizeof(float) * (size_t)a.n_atoms * a.C + 255) & ~(size_t)255));
  so2_status st;
  if ((st = fill_zero(dx, (int64_t)a.n_atoms * nc * a.C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dpos, (int64_t)a.n_atoms * 3, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dk, (int64_t)a.n_atoms * a.C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dw_q, (int64_t)a.C * a.C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dw_k, (int64_t)a.C * a.C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dw_rad, (int64_t)a.K * a.C, stream)) != SO2_OK) return st;
  if ((st = fill_zero(dw_so2, so2_w1_offset(a.L, a.C, a.L + 1), stream)) != SO2_OK) return st;
  hipLaunchKernelGGL(generators_kernel, dim3(1), dim3(64), 0, stream, gen, gen + 3 * wig_total(a.L), a.L);
  SO2_CHECK_LAUNCH();
  if (a.n_targets > 0) {
    BwdParams P{};
    P.pos = a.pos;
    P.row_ptr = a.row_ptr;
    P.col = a.col;
    P.x = a.x;
    P.w_q = a.w_q;
    P.w_k = a.w_k;
    P.w_rad = a.w_rad;
    P.w_so2 = a.w_so2;
    P.dy = dy;
    P.q = a.q;
    P.k = a.k;
    P.gen = gen;
    P.dq = dq;
    P.dk = dk;
    P.dx = dx;
    P.dpos = dpos;
    P.dw_rad = dw_rad;
    P.dw_so2 = dw_so2;
    P.n_atoms = a.n_atoms;
    P.n_targets = a.n_targets;
    P.L = a.L;
    P.C = a.C;
    P.H = a.H;
    P.K = a.K;
    P.p = a.p;
    P.cutoff = a.cutoff;
    P.flags = a.flags;
    P.periodic = a.periodic;
    for (int d = 0; d < 3; ++d) P.box[d] = a.box[d];
    const size_t smem = sizeof(float) * (size_t)BwdLds(a.L, a.C, a.H, a.K).total;
    if (a.dtype == SO2_BF16) {
      SO2_CHECK(hipFuncSetAttribute((const void*)attn_bwd_kernel<uint16_t>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem));
      hipLaunchKernelGGL(attn_bwd_kernel<uint16_t>, dim3(a.n_targets), dim3(kBwdThreads), smem, stream, P);
    } else {
      SO2_CHECK(hipFuncSetAttribute((const void*)attn_bwd_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)smem));
      hipLaunchKernelGGL(attn_bwd_kernel<float>, dim3(a.n_targets), dim3(kBwdThreads), smem, stream, P);
    }
    SO2_CHECK_LAUNCH();
  }
  // the projections of the l = 0 slice
  const int64_t nxc = (int64_t)a.n_atoms * a.C;
  const unsigned gdx = (unsigned)((nxc + 255) / 256);
  const unsigned gw = (unsigned)(((int64_t)a.C * a.C + 255) / 256);
  if (a.dtype == SO2_BF16) {
    hipLaunchKernelGGL(proj_bwd_dx_kernel<uint16_t>, dim3(gdx), dim3(256), 0, stream, dq, dk, a.w_q, a.w_k, dx,
                       a.n_atoms, a.n_targets, nc, a.C);
    if (dw_q && a.n_targets > 0)
      hipLaunchKernelGGL(proj_bwd_dw_kernel<uint16_t>, dim3(gw, (a.n_targets + kProjAtoms - 1) / kProjAtoms),
                         dim3(256), 0, stream, a.x, dq, dw_q, a.n_targets, nc, a.C);
    if (dw_k)
      hipLaunchKernelGGL(proj_bwd_dw_kernel<uint16_t>, dim3(gw, (a.n_atoms + kProjAtoms - 1) / kProjAtoms),
                         dim3(256), 0, stream, a.x, dk, dw_k, a.n_atoms, nc, a.C);
  } else {
    hipLaunchKernelGGL(proj_bwd_dx_kernel<float>, dim3(gdx), dim3(256), 0, stream, dq, dk, a.w_q, a.w_k, dx,
                       a.n_atoms, a.n_targets, nc, a.C);
    if (dw_q && a.n_targets > 0)
      hipLaunchKernelGGL(proj_bwd_dw_kernel<float>, dim3(gw, (a.n_targets + kProjAtoms - 1) / kProjAtoms), dim3(256),
                         0, stream, a.x, dq, dw_q, a.n_targets, nc, a.C);
    if (dw_k)
      hipLaunchKernelGGL(proj_bwd_dw_kernel<float>, dim3(gw, (a.n_atoms + kProjAtoms - 1) / kProjAtoms), dim3(256),
                         0, stream, a.x, dk, dw_k, a.n_atoms, nc, a.C);
  }
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

}  // namespace so2
