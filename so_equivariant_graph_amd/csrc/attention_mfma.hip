// Fused SO(2) equivariant graph attention forward on gfx950 MFMA (bf16 in,
// fp32 accumulate).
//
// The method ("E2Former-V2: On-the-Fly Equivariant Attention with Linear
// Activation Memory", technical summary, sections 2.1 and 2.2; envelope in
// numerator and denominator from "EquiformerV3: Scaling Efficient, Expressive, and General SE(3)-Equivariant
// Graph Attention Transformers", technical summary, section
// 2.B.3): for every target atom stream its neighbours, rotate each
// neighbour's irreps into the edge frame, gate per channel, apply one linear
// map per |m|, rotate back, weight with the envelope-gated softmax and sum.
// No per-edge tensor leaves the workgroup.
//
// The per-m map is a dense contraction over channels and degrees shared by
// every edge, so it runs as GEMMs on the matrix cores
// (v_mfma_f32_16x16x32_bf16):
//
//   edges are the M dimension: a chunk holds up to 64 consecutive edges of
//   the CSR (4 row tiles of 16), crossing target boundaries;
//   for block m the A operand is the rotated, gated input rows (l', +-m) of
//   those edges, built on the vector ALUs from x_j and the edge's Wigner-D
//   rows and staged through LDS in bf16; the B operand is W0 (m = 0) or
//   W1_m / W2_m read straight from the caller's row-major [out][in] weights
//   (8 consecutive bf16 of one row per lane, one 16-byte load);
//   m >= 1 is the complex product (W1 + i W2)(xt_+ + i xt_-): four real MFMAs
//   per tile pair, the minus sign carried by negating the xt_- operand.
//
// Rotating back and summing over neighbours is a second, small GEMM: for
// output degree l the target accumulator rows are (l, target slot, m'), its
// K index is (edge, +-m) and its A operand holds D^l_e[+-m][m'] where edge e
// belongs to that target (0 elsewhere); its B operand is the weighted output
// of the first GEMM, which is already in the right lane layout (the K order
// follows the accumulator layout), so it is only scaled and rounded to bf16.
// The target accumulators live in LDS in the MFMA C layout.
//
// Workgroup: 8 waves (512 lanes), wave w owns output channels
// [16w, 16w+16).  Each workgroup takes a run of consecutive target atoms
// holding about the same number of edges as every other workgroup; its
// edges are processed in chunks of at most 64 edges whose targets span at
// most 4 consecutive indices (4 accumulator slots, slot = target mod 4); a
// target whose edges continue into the next chunk keeps its slot, a target
// whose last edge is in the chunk is written out and its slot cleared.
//
// Softmax weights come from a statistics pass (attn_stats_kernel): for every
// target and head the running maximum and the normaliser
// sum_j u_ij exp(z_ij - max), accumulated online over the neighbours, so the
// fused kernel applies final weights and never rescales its accumulators.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "wigner.h"

namespace so2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kC = 128;               // channels
constexpr int kWaves = kC / 16;       // 8 waves, 16 output channels each
constexpr int kThreads = kWaves * 64;
constexpr int kM = 64;                // edges per chunk
constexpr int kRT = kM / 16;          // row tiles
constexpr int kSlots = 4;             // targets live in one chunk
constexpr int kEdgesPerGroup = 384;   // edges per workgroup (about six chunks)
constexpr int kKC = 64;               // channels per K chunk (2 MFMA K steps)
constexpr int kApad = kKC + 8;        // LDS row pitch of the A chunk, bf16
constexpr int kMaxHeads = 16;
constexpr int kGpad = kC + 8;         // LDS row pitch of the radial gate, bf16
constexpr int kMaxDeg = 2;            // output degrees per pass for m >= 1

struct MfmaParams {
  const float* pos;
  const int32_t* row_ptr;
  const int32_t* col;
  const uint16_t* x;
  const uint16_t* w_rad;
  const uint16_t* w_so2;
  const float* q;
  const float* k;
  float* stat_max;  // [n_targets][H]
  float* stat_inv;  // [n_targets][H]
  float* y;
  uint32_t x_bytes;  // extent of x for its buffer descriptor (< 4 GiB)
  uint32_t w_bytes;  // extent of w_so2
  int32_t n_targets, H, K, p;
  float cutoff;
  uint32_t flags;
  int32_t periodic;
  float box[3];
};

__device__ inline float bf_lo(unsigned int u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(unsigned int u) { return __uint_as_float(u & 0xffff0000u); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// Two floats to packed bf16 (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ inline unsigned int pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer descriptor (gfx9 family: dword3 = 0x00020000).  Loads through
// it take one 32-bit VGPR offset and return 0 past num_records bytes.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ inline void edge_vec(const MfmaParams& P, int i, int j, float* r) {
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    float v = P.pos[3 * (int64_t)j + d] - P.pos[3 * (int64_t)i + d];
    if (P.periodic) v = v - P.box[d] * rintf(v / P.box[d]);
    r[d] = v;
  }
}

// ---------------------------------------------------------------- statistics

// One wave per target: lanes walk the neighbours, each keeps an online
// (max, normaliser) pair per head; the wave then combines the pairs.
__global__ void __launch_bounds__(256) attn_stats_kernel(MfmaParams P, int C) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= P.n_targets) return;
  const int e0 = P.row_ptr[t], e1 = P.row_ptr[t + 1];
  const int H = P.H, d = C / H;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  for (int h = 0; h < H; ++h) {
    float m = -INFINITY, s = 0.0f;
    for (int e = e0 + lane; e < e1; e += 64) {
      const int j = P.col[e];
      float r[3];
      edge_vec(P, t, j, r);
      const float rho = sqrtf(r[0] * r[0] + r[1] * r[1] + r[2] * r[2]);
      const float u = envelope_u(rho / P.cutoff, P.p);
      float z = 0.0f;
      for (int c = h * d; c < (h + 1) * d; ++c) z += P.q[(int64_t)t * C + c] * P.k[(int64_t)j * C + c];
      z *= inv_sqrt_d;
      if (z > m) {
        s = s * expf(m - z) + u;
        m = z;
      } else {
        s += u * expf(z - m);
      }
    }
    float M = m;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    float part = (m == -INFINITY) ? 0.0f : s * expf(m - M);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) {
      P.stat_max[(int64_t)t * H + h] = M;
      P.stat_inv[(int64_t)t * H + h] = part > 0.0f ? 1.0f / part : 0.0f;
    }
  }
}

// ---------------------------------------------------------------- layout

template <int L>
struct Cfg {
  static constexpr int NC = (L + 1) * (L + 1);
  static constexpr int WT = wig_total(L);
  // target accumulator rows (l, slot, m') packed: kSlots l^2 + slot (2l+1) + m' + l
  static constexpr int TROWS = kSlots * NC;
  static constexpr int TT = (TROWS + 15) / 16;  // 16-row MFMA tiles
};

struct Smem {
  int rp[kSlots + 2];   // row_ptr[t_first .. t_first + kSlots]
  int flush_t[kSlots];  // target written out from each slot after this chunk, or -1
  int row_j[kM];
  int row_slot[kM];
};

template <int L>
struct Lds {
  static constexpr size_t kHdr = (sizeof(Smem) + 15) & ~(size_t)15;
  static constexpr size_t kD = kHdr;                                    // float [kM][WT]
  static constexpr size_t kG = kD + sizeof(float) * kM * Cfg<L>::WT;    // bf16 [kM][kGpad]
  static constexpr size_t kW = kG + sizeof(uint16_t) * kM * kGpad;      // float [kM][kMaxHeads]
  static constexpr size_t kA = kW + sizeof(float) * kM * kMaxHeads;     // bf16 [2][2][kM][kApad]
  static constexpr size_t kAbuf = sizeof(uint16_t) * 2 * kM * kApad;    // one buffer, both signs
  static constexpr size_t kT = kA + 2 * kAbuf;                          // f32x4 [TT][kWaves][64]
  static constexpr size_t kTotal = kT + sizeof(f32x4) * Cfg<L>::TT * kWaves * 64;
};

// Target accumulator tile ot of wave w, in the MFMA C layout (lane, 4 rows).
template <int L>
__device__ inline f32x4* tacc_tile(char* smem, int ot, int wave) {
  return (f32x4*)(smem + Lds<L>::kT) + (ot * kWaves + wave) * 64;
}

// Edge er of the chunk: its target t (one of the slots' targets), source j
// and minimum-image vector r_ij = p_j - p_t.
__device__ inline void row_edge(const MfmaParams& P, const Smem& S, int er, int t_first, int& t, int& j,
                                float* rv) {
  int s = 0;
  while (s + 1 < kSlots && S.rp[s + 1] <= er) ++s;
  t = t_first + s;
  j = P.col[er];
  edge_vec(P, t, j, rv);
}

// ---------------------------------------------------------------- A operand

// Build one A chunk: rows of 64 edges, 64 channels [cbase, cbase+64) of
// degree lp, for +m and (m > 0) -m:  a[r][c] = g_r[c] sum_b D^lp_r[+-m][b] x_j[(lp,b)][c].
// Lane (r = tid / 8, 8 channels at cbase + 8 (tid % 8)).  gen_load issues the
// 2lp+1 gathers of x_j back to back (one 16-byte load each); gen_store
// combines them with the edge's Wigner-D rows and the radial gate.
constexpr int kMaxComp = 2 * 4 + 1;  // 2 L + 1 for L <= 4

__device__ inline void gen_load(__amdgpu_buffer_rsrc_t xrs, const Smem& S, int NC, int lp, int cbase,
                                u32x4 (&xr)[kMaxComp]) {
  const int tid = threadIdx.x;
  const int r = tid >> 3;
  const int c = cbase + 8 * (tid & 7);
  const int j = S.row_j[r];
  const int n = 2 * lp + 1;
  const uint32_t voff = (((uint32_t)(j < 0 ? 0 : j) * NC + lp * lp) * kC + c) * 2u;
#pragma unroll
  for (int b = 0; b < kMaxComp; ++b)
    if (b < n && j >= 0) xr[b] = buffer_load16(xrs, voff + b * kC * 2, 0);
}

template <int L, int NS>
__device__ inline void gen_store(char* smem, int m, int lp, int cbase, const u32x4 (&xr)[kMaxComp],
                                 uint16_t* abuf) {
  const Smem& S = *(const Smem*)smem;
  const float* sD = (const float*)(smem + Lds<L>::kD);
  const uint16_t* sG = (const uint16_t*)(smem + Lds<L>::kG);
  const int tid = threadIdx.x;
  const int r = tid >> 3;
  const int cg = tid & 7;
  const int c = cbase + 8 * cg;
  const int j = S.row_j[r];
  const int n = 2 * lp + 1;
  float ap[8], am[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) ap[q] = am[q] = 0.0f;
  if (j >= 0) {
    const float* Dl = sD + r * Cfg<L>::WT + wig_offset(lp);
    const float* dp = Dl + (lp + m) * n;
    const float* dm = Dl + (lp - m) * n;
#pragma unroll
    for (int b = 0; b < kMaxComp; ++b) {
      if (b < n) {
        const u32x4 v = xr[b];
        const float xv[8] = {bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y),
                             bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w)};
        const float wp = dp[b];
#pragma unroll
        for (int q = 0; q < 8; ++q) ap[q] += wp * xv[q];
        if (NS > 1) {
          const float wm = dm[b];
#pragma unroll
          for (int q = 0; q < 8; ++q) am[q] += wm * xv[q];
        }
      }
    }
    const u32x4 gv = *(const u32x4*)(sG + r * kGpad + c);
    const float g[8] = {bf_lo(gv.x), bf_hi(gv.x), bf_lo(gv.y), bf_hi(gv.y),
                        bf_lo(gv.z), bf_hi(gv.z), bf_lo(gv.w), bf_hi(gv.w)};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ap[q] *= g[q];
      am[q] *= g[q];
    }
  }
  u32x4 op;
  op.x = pack_bf16x2(ap[0], ap[1]);
  op.y = pack_bf16x2(ap[2], ap[3]);
  op.z = pack_bf16x2(ap[4], ap[5]);
  op.w = pack_bf16x2(ap[6], ap[7]);
  *(u32x4*)(abuf + r * kApad + 8 * cg) = op;
  if (NS > 1) {
    u32x4 om;
    om.x = pack_bf16x2(am[0], am[1]);
    om.y = pack_bf16x2(am[2], am[3]);
    om.z = pack_bf16x2(am[4], am[5]);
    om.w = pack_bf16x2(am[6], am[7]);
    *(u32x4*)(abuf + (kM + r) * kApad + 8 * cg) = om;
  }
}

// ---------------------------------------------------------------- main GEMM

// K loop of one pass: stream A chunks (degree lp, 64 channels, +m and for
// m > 0 also -m) through double-buffered LDS and accumulate
//   m = 0:  acc[d][0] += xt_0 W0^T
//   m > 0:  acc[d][0] += xt_+ W1^T - xt_- W2^T,  acc[d][1] += xt_+ W2^T + xt_- W1^T
// for output degrees lo .. lo+nd-1 (nd <= ND) of this wave's 16 channels.
// The K steps (32 inputs each, two per A chunk) run as one flat loop; the B
// fragments of step s+1 are loaded before the MFMAs of step s.
template <int L, int ND, int NS>
__device__ inline void load_b(__amdgpu_buffer_rsrc_t wrs, uint32_t w1_byte, uint32_t w2_byte, int KM,
                              int m, int lo, int nd, int s, u32x4 (&b1)[ND], u32x4 (&b2)[ND]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = s >> 1;
  const int kin = (q / (kC / kKC)) * kC + kKC * (q % (kC / kKC)) + 32 * (s & 1) + 8 * (lane >> 4);
#pragma unroll
  for (int di = 0; di < ND; ++di) {
    if (di < nd) {
      const int row = (lo + di - m) * kC + 16 * wave + (lane & 15);
      const uint32_t voff = (uint32_t)(row * KM + kin) * 2u;
      b1[di] = buffer_load16(wrs, voff, w1_byte);
      if (NS > 1) b2[di] = buffer_load16(wrs, voff, w2_byte);
    }
  }
}

template <int L, int ND, int NS>
__device__ inline void main_gemm(const MfmaParams& P, char* smem, int m, int lo, int nd,
                                 f32x4 (&acc)[ND][NS][kRT]) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  uint16_t* abase = (uint16_t*)(smem + Lds<L>::kA);
  const int KM = (L + 1 - m) * kC;
  const int NQ = (L + 1 - m) * (kC / kKC);
  const uint32_t w1_byte = (uint32_t)(m == 0 ? 0 : so2_w1_offset(L, kC, m)) * 2u;
  const uint32_t w2_byte = w1_byte + (uint32_t)(KM * KM) * 2u;
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(P.w_so2, P.w_bytes);
  const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(P.x, P.x_bytes);

  const Smem& S = *(const Smem*)smem;
  constexpr int NC = Cfg<L>::NC;
  u32x4 b1[ND], b2[ND], n1[ND], n2[ND];
  u32x4 xr[kMaxComp];
  load_b<L, ND, NS>(wrs, w1_byte, w2_byte, KM, m, lo, nd, 0, b1, b2);
  gen_load(xrs, S, NC, m, 0, xr);
  gen_store<L, NS>(smem, m, m, 0, xr, abase);
  __syncthreads();
  for (int s = 0; s < 2 * NQ; ++s) {
    const int q = s >> 1;
    const int ks = s & 1;
    const uint16_t* abuf = abase + (q & 1) * (2 * kM * kApad);
    const int lq = m + (q + 1) / (kC / kKC);      // next A chunk
    const int cq = kKC * ((q + 1) % (kC / kKC));
    // gathers for the next A chunk go out first; they land during this chunk's MFMAs
    if (ks == 0 && q + 1 < NQ) gen_load(xrs, S, NC, lq, cq, xr);
    if (s + 1 < 2 * NQ) load_b<L, ND, NS>(wrs, w1_byte, w2_byte, KM, m, lo, nd, s + 1, n1, n2);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int off = (16 * rt + l16) * kApad + 32 * ks + 8 * g4;
      const u32x4 ap = *(const u32x4*)(abuf + off);
      if (NS == 1) {
#pragma unroll
        for (int di = 0; di < ND; ++di)
          acc[di][0][rt] = mfma(as_bf16x8(ap), as_bf16x8(b1[di]), acc[di][0][rt]);
      } else {
        const u32x4 am = *(const u32x4*)(abuf + kM * kApad + off);
        const u32x4 amn = am ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
        for (int di = 0; di < ND; ++di) {
          if (di < nd) {
            acc[di][0][rt] = mfma(as_bf16x8(ap), as_bf16x8(b1[di]), acc[di][0][rt]);
            acc[di][0][rt] = mfma(as_bf16x8(amn), as_bf16x8(b2[di]), acc[di][0][rt]);
            acc[di][NS - 1][rt] = mfma(as_bf16x8(ap), as_bf16x8(b2[di]), acc[di][NS - 1][rt]);
            acc[di][NS - 1][rt] = mfma(as_bf16x8(am), as_bf16x8(b1[di]), acc[di][NS - 1][rt]);
          }
        }
      }
    }
    if (ks == 1 && q + 1 < NQ) gen_store<L, NS>(smem, m, lq, cq, xr, abase + ((q + 1) & 1) * (2 * kM * kApad));
#pragma unroll
    for (int di = 0; di < ND; ++di) {
      b1[di] = n1[di];
      b2[di] = n2[di];
    }
    if (ks == 1) __syncthreads();
  }
}

// ---------------------------------------------------------------- rotate back

// Rotate back and sum over neighbours for output degree l of block m:
//   T[l] += A'(D, slots) x B'(w * yt).
// yt[s][rt] is the main GEMM accumulator of this degree (s = 0: +m or m = 0,
// s = 1: -m), lane rows 4 (lane/16) + i of row tile rt, column lane % 16.
// B' is yt scaled by the lane's head weight and rounded to bf16, packed so
// that K index 8 g + jj of lane group g is
//   m > 0:  edge 16 st + 4 g + (jj & 3), sign + for jj < 4, - otherwise
//   m = 0:  edge 16 (2 st + jj / 4) + 4 g + (jj & 3);
// A' row R of the accumulator (R = kSlots l^2 + slot (2l+1) + m' + l) holds
// D^l_e[l +- m][m' + l] in the same K order when edge e belongs to that
// slot's target, 0 otherwise (and 0 on rows of other degrees).  A' does not
// depend on the output channels, so the whole workgroup builds it once per
// pass into LDS (aprime_build) and every wave reads it from there.

__device__ inline int deg_tiles(int l) {
  return (kSlots * (l + 1) * (l + 1) - 1) / 16 - (kSlots * l * l) / 16 + 1;
}

// A' fragments of a pass (degrees lo .. lo+nd-1), in the order
// (degree, tile, K step), 64 lanes x 16 bytes each, written to frag.
template <int L>
__device__ inline void aprime_build(char* smem, int m, int lo, int nd, u32x4* frag) {
  const Smem& S = *(const Smem*)smem;
  const float* sD = (const float*)(smem + Lds<L>::kD);
  const int steps = m == 0 ? kRT / 2 : kRT;
  int total = 0;
  for (int di = 0; di < nd; ++di) total += deg_tiles(lo + di) * steps;
  for (int idx = threadIdx.x; idx < total * 64; idx += kThreads) {
    int f = idx >> 6;
    const int lane = idx & 63;
    int l = lo;
    while (f >= deg_tiles(l) * steps) {
      f -= deg_tiles(l) * steps;
      ++l;
    }
    const int ot = (kSlots * l * l) / 16 + f / steps;
    const int st = f % steps;
    const int n = 2 * l + 1;
    const int r0 = kSlots * l * l, r1 = kSlots * (l + 1) * (l + 1);
    const int R = 16 * ot + (lane & 15);
    const bool mine = R >= r0 && R < r1;
    const int oslot = mine ? (R - r0) / n : -1;
    const int omp = mine ? (R - r0) - oslot * n : 0;
    const int g4 = lane >> 4;
    float av[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      int r, srow;
      if (m > 0) {
        r = 16 * st + 4 * g4 + (jj & 3);
        srow = (jj < 4) ? (l + m) : (l - m);
      } else {
        r = 16 * (2 * st + (jj >> 2)) + 4 * g4 + (jj & 3);
        srow = l;
      }
      av[jj] = S.row_slot[r] == oslot ? sD[r * Cfg<L>::WT + wig_offset(l) + srow * n + omp] : 0.0f;
    }
    u32x4 a;
    a.x = pack_bf16x2(av[0], av[1]);
    a.y = pack_bf16x2(av[2], av[3]);
    a.z = pack_bf16x2(av[4], av[5]);
    a.w = pack_bf16x2(av[6], av[7]);
    frag[idx] = a;
  }
}

template <int L, int NS>
__device__ inline void rot_back(char* smem, const f32x4 (&yt)[NS][kRT], int l, int head,
                                const u32x4* frag) {
  const float* sW = (const float*)(smem + Lds<L>::kW);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g4 = lane >> 4;
  constexpr bool M0 = NS == 1;
  u32x4 bq[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    float w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w4[i] = sW[(16 * rt + 4 * g4 + i) * kMaxHeads + head];
    if (!M0) {
      const f32x4 yp = yt[0][rt], ym = yt[NS - 1][rt];
      bq[rt].x = pack_bf16x2(yp[0] * w4[0], yp[1] * w4[1]);
      bq[rt].y = pack_bf16x2(yp[2] * w4[2], yp[3] * w4[3]);
      bq[rt].z = pack_bf16x2(ym[0] * w4[0], ym[1] * w4[1]);
      bq[rt].w = pack_bf16x2(ym[2] * w4[2], ym[3] * w4[3]);
    } else {
      const f32x4 y0 = yt[0][rt];
      const unsigned int lo01 = pack_bf16x2(y0[0] * w4[0], y0[1] * w4[1]);
      const unsigned int lo23 = pack_bf16x2(y0[2] * w4[2], y0[3] * w4[3]);
      if ((rt & 1) == 0) {
        bq[rt].x = lo01;
        bq[rt].y = lo23;
      } else {
        bq[rt - 1].z = lo01;
        bq[rt - 1].w = lo23;
      }
    }
  }
  constexpr int kSteps = M0 ? kRT / 2 : kRT;
  const int ot0 = (kSlots * l * l) / 16;
  const int nt = deg_tiles(l);
  for (int q = 0; q < nt; ++q) {
    f32x4* tile = tacc_tile<L>(smem, ot0 + q, wave);
    f32x4 tv = tile[lane];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const u32x4 a = frag[(q * kSteps + st) * 64 + lane];
      tv = mfma(as_bf16x8(a), as_bf16x8(bq[M0 ? 2 * st : st]), tv);
    }
    tile[lane] = tv;
  }
}

// ---------------------------------------------------------------- passes

// One pass: block m, output degrees lo .. lo+nd-1 (nd <= ND): main GEMM,
// then the A' fragments, then the rotate-back GEMM of each degree.
template <int L, int ND, int NS>
__device__ inline void pass(const MfmaParams& P, char* smem, int m, int lo, int nd, int head) {
  f32x4 acc[ND][NS][kRT];
#pragma unroll
  for (int a = 0; a < ND; ++a)
#pragma unroll
    for (int b = 0; b < NS; ++b)
#pragma unroll
      for (int c = 0; c < kRT; ++c) acc[a][b][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  main_gemm<L, ND, NS>(P, smem, m, lo, nd, acc);  // ends with a barrier
  u32x4* frag = (u32x4*)(smem + Lds<L>::kA);       // the A chunks are dead now
  aprime_build<L>(smem, m, lo, nd, frag);
  __syncthreads();
  const int steps = NS == 1 ? kRT / 2 : kRT;
  int fbase = 0;
#pragma unroll
  for (int di = 0; di < ND; ++di) {
    if (di < nd) {
      rot_back<L, NS>(smem, acc[di], lo + di, head, frag + fbase * 64);
      fbase += deg_tiles(lo + di) * steps;
    }
  }
  __syncthreads();  // the next pass overwrites the fragments
}

// ---------------------------------------------------------------- flush

// Write every slot whose target finished in this chunk to y (whole 512-byte
// rows) and clear it.  Accumulator element (slot, comp, c) sits in tile
// R / 16 (R = kSlots l^2 + slot (2l+1) + comp - l^2) of wave c / 16, lane
// 16 ((R % 16) / 4) + c % 16, entry R % 4.
template <int L>
__device__ inline void flush_slots(char* smem, float* y) {
  constexpr int NC = Cfg<L>::NC;
  const Smem& S = *(const Smem*)smem;
  float* T = (float*)(smem + Lds<L>::kT);
  for (int s = 0; s < kSlots; ++s) {
    const int t = S.flush_t[s];
    if (t < 0) continue;
    for (int a = threadIdx.x; a < NC * kC; a += kThreads) {
      const int comp = a / kC, c = a % kC;
      const int l = (int)sqrtf((float)comp + 0.5f);
      const int R = kSlots * l * l + s * (2 * l + 1) + (comp - l * l);
      const int idx = (((R >> 4) * kWaves + (c >> 4)) * 64 + 16 * ((R & 15) >> 2) + (c & 15)) * 4 + (R & 3);
      y[(int64_t)t * NC * kC + a] = T[idx];
      T[idx] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------- kernel

// First target of group g: the smallest t with row_ptr[t] - row_ptr[0] >=
// g E / n_groups (E = edges of all targets); group n_groups starts at
// n_targets.  Binary search, uniform across the workgroup.
__device__ inline int group_start(const MfmaParams& P, int g, int n_groups) {
  if (g >= n_groups) return P.n_targets;
  const int e0 = P.row_ptr[0];
  const int64_t E = (int64_t)P.row_ptr[P.n_targets] - e0;
  const int64_t goal = e0 + (E * g) / n_groups;
  int lo = 0, hi = P.n_targets;  // answer in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)P.row_ptr[mid] >= goal) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

template <int L>
__global__ void __launch_bounds__(kThreads) attn_mfma_kernel(MfmaParams P, int n_groups) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Smem& S = *(Smem*)smem;
  float* sD = (float*)(smem + Lds<L>::kD);
  uint16_t* sG = (uint16_t*)(smem + Lds<L>::kG);
  float* sW = (float*)(smem + Lds<L>::kW);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  constexpr int NC = Cfg<L>::NC;

  // Workgroup -> group of consecutive targets holding about E / n_groups
  // edges (group g starts at the first target whose edges start at or after
  // g E / n_groups), contiguous per XCD: workgroups are dispatched to the 8
  // XCDs round robin, and neighbouring groups share neighbours in L2.
  const int b = blockIdx.x;
  const int per = n_groups / 8, rem = n_groups % 8;
  const int xcd = b % 8, idx = b / 8;
  const int grp = xcd * per + min(xcd, rem) + idx;
  const int t_begin = group_start(P, grp, n_groups);
  const int t_end = group_start(P, grp + 1, n_groups);

  // targets without neighbours: y = 0
  for (int a = tid; a < (t_end - t_begin) * NC * kC; a += kThreads) {
    const int t = t_begin + a / (NC * kC);
    if (P.row_ptr[t] == P.row_ptr[t + 1]) P.y[(int64_t)t * NC * kC + a % (NC * kC)] = 0.0f;
  }
  for (int a = tid; a < Cfg<L>::TT * kWaves * 64; a += kThreads)
    ((f32x4*)(smem + Lds<L>::kT))[a] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int e_end = P.row_ptr[t_end];
  int e = P.row_ptr[t_begin];
  int t_cur = t_begin;
  const int H = P.H;
  const int dh = kC / H;
  const int head = (16 * wave + (tid & 15)) / dh;
  const float inv_sqrt_d = 1.0f / sqrtf((float)dh);
  const float rc = P.cutoff;

  while (e < e_end) {
    while (P.row_ptr[t_cur + 1] <= e) ++t_cur;  // target of edge e
    const int t_first = t_cur;
    const int t_lim = min(t_first + kSlots, t_end);
    const int e_stop = min(min(e + kM, e_end), P.row_ptr[t_lim]);
    const int nrows = e_stop - e;

    // ---- phase A: per-edge setup
    if (tid <= kSlots) S.rp[tid] = P.row_ptr[min(t_first + tid, t_end)];
    __syncthreads();
    if (tid < kSlots) {
      int sl = 0;  // target of the chunk's last edge: t_first + sl
      while (sl + 1 < kSlots && S.rp[sl + 1] <= e_stop - 1) ++sl;
      const int t = t_first + ((tid - t_first % kSlots + kSlots) % kSlots);
      S.flush_t[tid] = (t <= t_first + sl && S.rp[t - t_first + 1] <= e_stop) ? t : -1;
    }
    if (tid < kM) {
      // wave 0: one edge per lane: metadata, frame and all Wigner-D blocks
      const int r = tid;
      if (r < nrows) {
        int t, j;
        float rv[3];
        row_edge(P, S, e + r, t_first, t, j, rv);
        const float rho = sqrtf(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]);
        S.row_j[r] = j;
        S.row_slot[r] = t % kSlots;
        const float inv = rho > 0.0f ? 1.0f / rho : 0.0f;
        float R[9];
        edge_frame(rv[0] * inv, rv[1] * inv, rv[2] * inv, R);
        wigner_blocks_unrolled<L>(R, sD + r * Cfg<L>::WT);
      } else {
        S.row_j[r] = -1;
        S.row_slot[r] = -2;  // matches no slot
      }
    } else {
      // waves 1..7: radial gates (64 rows x 8 groups of 16 channels), then
      // the softmax weights (64 rows x kMaxHeads)
      for (int it = tid - kM; it < kM * (kC / 16) + kM * kMaxHeads; it += kThreads - kM) {
        if (it < kM * (kC / 16)) {
          const int r = it / (kC / 16), c0 = 16 * (it % (kC / 16));
          float gv[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) gv[q] = 0.0f;
          if (r < nrows) {
            if (P.flags & SO2_FLAG_NO_RADIAL) {
#pragma unroll
              for (int q = 0; q < 16; ++q) gv[q] = 1.0f;
            } else {
              int t, j;
              float rv[3];
              row_edge(P, S, e + r, t_first, t, j, rv);
              const float rho = sqrtf(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]);
              const float step = rc / (float)(P.K - 1);
              const float inv2s2 = 1.0f / (2.0f * step * step);
              for (int kk = 0; kk < P.K; ++kk) {
                const float dr = rho - step * (float)kk;
                const float phi = expf(-dr * dr * inv2s2);
                const uint16_t* wr = P.w_rad + (int64_t)kk * kC + c0;
                const u32x4 v0 = *(const u32x4*)wr;
                const u32x4 v1 = *(const u32x4*)(wr + 8);
                const float wv[16] = {bf_lo(v0.x), bf_hi(v0.x), bf_lo(v0.y), bf_hi(v0.y),
                                      bf_lo(v0.z), bf_hi(v0.z), bf_lo(v0.w), bf_hi(v0.w),
                                      bf_lo(v1.x), bf_hi(v1.x), bf_lo(v1.y), bf_hi(v1.y),
                                      bf_lo(v1.z), bf_hi(v1.z), bf_lo(v1.w), bf_hi(v1.w)};
#pragma unroll
                for (int q = 0; q < 16; ++q) gv[q] += phi * wv[q];
              }
              if (P.flags & SO2_FLAG_RBF_ENVELOPE) {
                const float u = envelope_u(rho / rc, P.p);
#pragma unroll
                for (int q = 0; q < 16; ++q) gv[q] *= u;
              }
            }
          }
          u32x4 g0, g1;
          g0.x = pack_bf16x2(gv[0], gv[1]);
          g0.y = pack_bf16x2(gv[2], gv[3]);
          g0.z = pack_bf16x2(gv[4], gv[5]);
          g0.w = pack_bf16x2(gv[6], gv[7]);
          g1.x = pack_bf16x2(gv[8], gv[9]);
          g1.y = pack_bf16x2(gv[10], gv[11]);
          g1.z = pack_bf16x2(gv[12], gv[13]);
          g1.w = pack_bf16x2(gv[14], gv[15]);
          *(u32x4*)(sG + r * kGpad + c0) = g0;
          *(u32x4*)(sG + r * kGpad + c0 + 8) = g1;
        } else {
          const int pr = it - kM * (kC / 16);
          const int r = pr / kMaxHeads, h = pr % kMaxHeads;
          float wv = 0.0f;
          if (r < nrows && h < H) {
            int t, j;
            float rv[3];
            row_edge(P, S, e + r, t_first, t, j, rv);
            const float rho = sqrtf(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]);
            const float u = envelope_u(rho / rc, P.p);
            float z = 0.0f;
            for (int c = h * dh; c < (h + 1) * dh; ++c) z += P.q[(int64_t)t * kC + c] * P.k[(int64_t)j * kC + c];
            z *= inv_sqrt_d;
            wv = u * expf(z - P.stat_max[(int64_t)t * H + h]) * P.stat_inv[(int64_t)t * H + h];
          }
          sW[r * kMaxHeads + h] = wv;
        }
      }
    }
    __syncthreads();

    // ---- phase B: per-m GEMMs and the rotate-back GEMMs
#pragma nounroll
    for (int lo = 0; lo <= L; lo += 3) pass<L, 3, 1>(P, smem, 0, lo, min(3, L + 1 - lo), head);
#pragma nounroll
    for (int m = 1; m <= L; ++m) {
#pragma nounroll
      for (int lo = m; lo <= L; lo += kMaxDeg) pass<L, kMaxDeg, 2>(P, smem, m, lo, min(kMaxDeg, L + 1 - lo), head);
    }

    // ---- phase D: write out targets whose last edge is in this chunk
    flush_slots<L>(smem, P.y);
    e = e_stop;
    __syncthreads();
  }
}

// Workgroups: about kEdgesPerGroup edges each, rounded up to a whole number
// of waves of workgroups over the device's compute units (one per CU).
template <int L>
so2_status launch_L(const MfmaParams& P, int64_t n_edges, hipStream_t stream) {
  int dev = 0, n_cu = 256;
  SO2_CHECK(hipGetDevice(&dev));
  SO2_CHECK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  int64_t want = (n_edges + kEdgesPerGroup - 1) / kEdgesPerGroup;
  want = ((want + n_cu - 1) / n_cu) * n_cu;
  const int n_groups = (int)std::max<int64_t>(1, std::min<int64_t>(want, P.n_targets));
  const size_t smem = Lds<L>::kTotal;
  static_assert(Lds<L>::kTotal <= 160 * 1024, "LDS budget");
  SO2_CHECK(hipFuncSetAttribute((const void*)attn_mfma_kernel<L>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem));
  hipLaunchKernelGGL(attn_mfma_kernel<L>, dim3(n_groups), dim3(kThreads), smem, stream, P, n_groups);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

MfmaParams make_params(const AttnArgs& a) {
  MfmaParams P{};
  P.pos = a.pos;
  P.row_ptr = a.row_ptr;
  P.col = a.col;
  P.x = (const uint16_t*)a.x;
  P.w_rad = (const uint16_t*)a.w_rad;
  P.w_so2 = (const uint16_t*)a.w_so2;
  P.q = a.q;
  P.k = a.k;
  float* stats = (float*)a.scratch;
  P.stat_max = stats;
  P.stat_inv = stats + (size_t)a.n_targets * a.H;
  P.y = a.y;
  P.x_bytes = (uint32_t)((uint64_t)a.n_atoms * (a.L + 1) * (a.L + 1) * kC * 2);
  P.w_bytes = (uint32_t)(so2_w1_offset(a.L, kC, a.L + 1) * 2);
  P.n_targets = a.n_targets;
  P.H = a.H;
  P.K = a.K;
  P.p = a.p;
  P.cutoff = a.cutoff;
  P.flags = a.flags;
  P.periodic = a.periodic;
  for (int d = 0; d < 3; ++d) P.box[d] = a.box[d];
  return P;
}

}  // namespace

bool mfma_supported(int L, int C, int H, int n_atoms) {
  // x is addressed through a 32-bit buffer descriptor
  const uint64_t x_bytes = (uint64_t)n_atoms * (L + 1) * (L + 1) * C * 2;
  return C == kC && L >= 1 && L <= 4 && H >= 1 && H <= kMaxHeads && C % H == 0 &&
         x_bytes < 0xffffffffull;
}

bool mfma_aligned(const AttnArgs& a) {
  return !(((uintptr_t)a.x & 15) || ((uintptr_t)a.w_so2 & 15) || ((uintptr_t)a.w_rad & 15));
}

size_t mfma_scratch_bytes(int n_targets, int H) { return sizeof(float) * 2 * (size_t)n_targets * H + 256; }

so2_status launch_attention_mfma_prep(const AttnArgs& a, hipStream_t stream) {
  if (a.n_targets == 0) return SO2_OK;
  const MfmaParams P = make_params(a);
  hipLaunchKernelGGL(attn_stats_kernel, dim3((a.n_targets + 3) / 4), dim3(256), 0, stream, P, kC);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

so2_status launch_attention_mfma(const AttnArgs& a, hipStream_t stream) {
  if (a.n_targets == 0) return SO2_OK;
  const MfmaParams P = make_params(a);
  switch (a.L) {
    case 1:
      return launch_L<1>(P, a.n_edges, stream);
    case 2:
      return launch_L<2>(P, a.n_edges, stream);
    case 3:
      return launch_L<3>(P, a.n_edges, stream);
    case 4:
      return launch_L<4>(P, a.n_edges, stream);
  }
  return SO2_ERR_UNSUPPORTED;
}

}  // namespace so2
