// Fused SO(2) equivariant graph attention forward on gfx950 MFMA (bf16 in,
// fp32 accumulate).
//
// The method ("E2Former-V2: On-the-Fly Equivariant Attention with Linear
// Activation Memory", technical summary, sections 2.1 and 2.2; envelope in
// numerator and denominator from "EquiformerV3: Scaling Efficient,
// Expressive, and General SE(3)-Equivariant Graph Attention Transformers",
// technical summary, section 2.B.3): for every target atom stream its
// neighbours, rotate each neighbour's irreps into the edge frame, gate per
// channel, apply one linear map per |m|, rotate back, weight with the
// envelope-gated softmax and sum.  No per-edge tensor leaves the workgroup.
//
// The per-m map is a dense contraction over channels and degrees shared by
// every edge, so it runs as GEMMs on the matrix cores
// (v_mfma_f32_16x16x32_bf16):
//
//   edges are the M dimension: a chunk holds up to 64 consecutive edges of
//   the CSR (4 row tiles of 16; 32 edges and 2 row tiles for L = 5, 6),
//   crossing target boundaries;
//   for block m the A operand is the rotated, gated input rows (l', +-m) of
//   those edges, built on the vector ALUs and staged through LDS in bf16,
//   one degree l' (128 channels, 4 K steps of 32) per A chunk;
//   the B operand is W0 (m = 0) or W1_m / W2_m, copied by the prologue from
//   the caller's row-major [out][in] weights into MFMA fragment order, so
//   that one 16-byte load per lane is a whole fragment;
//   m >= 1 is the complex product (W1 + i W2)(xt_+ + i xt_-): four real MFMAs
//   per tile pair, the minus sign applied by flipping W2's sign bits in
//   registers.
//
// The rotation into the edge frame, xt[(l', m)][c] = sum_b D^l'[m][b]
// x_j[(l', b)][c], runs on v_dot2_f32_bf16: a prologue kernel repacks x so
// that one dword holds the components b = 2p and 2p+1 of one channel
// (zero for the odd one out), and the Wigner-D rows are kept in LDS as the
// matching bf16 pairs, so each dot2 is two multiply-adds with no unpacking.
//
// Rotating back and summing over neighbours is a second, small GEMM: for
// output degree l the target accumulator rows are (l, target slot, m'), its
// K index is (edge, +-m) and its A operand holds D^l_e[+-m][m'] where edge e
// belongs to that target (0 elsewhere); its B operand is the weighted output
// of the first GEMM, which is already in the right lane layout (the K order
// follows the accumulator layout), so it is only scaled and rounded to bf16.
// The target accumulators stay in registers in the MFMA C layout.
//
// Workgroup: 8 waves (512 lanes), two per SIMD so that one wave's memory
// waits are covered by the other's MFMAs; wave w owns output channels
// [16w, 16w+16).  Each workgroup (one per compute unit) takes a run of
// consecutive target atoms holding about the same number of edge chunks as
// every other workgroup (scheduling kernels choose the runs); its edges are
// processed in
// chunks of at most 64 (32) edges whose targets span at most 4 consecutive
// indices (4 accumulator slots, slot = target mod 4); a target whose edges
// continue into the next chunk keeps its slot, a target whose last edge is
// in the chunk is written out and its slot cleared.
//
// Software pipeline: while the MFMAs consume A chunk q from one LDS buffer,
// every lane generates one quarter of the next A chunk per K step into the
// other buffer (its gathers issued one step ahead, its dot products after
// the step's MFMAs) and the B fragments of the next K step load; one
// barrier per A chunk.  Every pass
// (block m, a group of output degrees) is a compile-time instance, so its
// loop bounds, weight offsets and register tiles are constants, and it
// generates the first A chunk of the pass after it.
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
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kC = 128;               // channels
constexpr int kWaves = 8;             // two waves per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kNT = kC / (16 * kWaves);  // 16-column tiles per wave: wave w owns channels 16 kNT w ..
constexpr int kGR = 1;                // generator rows per lane and K step
constexpr int kMaxM = 64;             // largest chunk
constexpr int kSlots = 4;             // targets live in one chunk
constexpr int kKC = 128;              // channels per A chunk (one degree, 4 MFMA K steps)
constexpr int kMaxHeads = 16;
constexpr int kMaxRbf = 32;           // radial basis functions kept per edge in LDS

// Edges per chunk: 64 up to L = 4; 32 for L = 5, 6, where the Wigner-D
// rows, the A' fragments and the accumulators of 64 edges would not fit the
// 160 KB of LDS and the register file.
__host__ __device__ constexpr int chunk_edges(int L) { return L <= 4 ? 64 : 32; }

// Chunk geometry of degree L.  In every K step each lane generates GCH
// channels of one edge row of the next A chunk: GL lanes per row, so the
// GL lanes of a row read one contiguous 32-channel slice of x pairs.
template <int L>
struct Geo {
  static constexpr int M = chunk_edges(L);       // edges per chunk
  static constexpr int RT = M / 16;              // MFMA row tiles
  static constexpr int GL = kThreads / M;        // generator lanes per edge row
  static constexpr int GCH = 32 / GL;            // channels per generator lane and K step
  static constexpr int MP = L + 1 > 5 ? L + 1 : 5;  // component pairs per generator unit
  static constexpr int APLANE = M * kKC;         // one sign plane of an A chunk, bf16
  static constexpr int ABUF = 2 * APLANE;        // one A buffer (both signs), bf16
};
static_assert(kThreads == 8 * 64, "phase A maps the 512 lanes onto the edge rows of a chunk");

// Gather vector of a generator lane: its GCH channels of one x pair.
template <int G>
struct XVec;
template <>
struct XVec<4> {
  typedef u32x4 type;
};
template <>
struct XVec<2> {
  typedef u32x2 type;
};

// Component pairs: degree l has l + 1 pairs (2p, 2p+1), the last one padded
// with zero.  pair_off(l) = pairs of the degrees below l.
__host__ __device__ constexpr int pair_off(int l) { return l * (l + 1) / 2; }
// Wigner-D pair dwords of the degrees below l: sum_{k<l} (2k+1)(k+1).
__host__ __device__ constexpr int dpair_off(int l) {
  return l * (l - 1) * (2 * l - 1) / 3 + 3 * l * (l - 1) / 2 + l;
}
__host__ __device__ constexpr int64_t w1_offset(int L, int m) {
  int64_t off = (int64_t)(L + 1) * kC * (L + 1) * kC;
  for (int mu = 1; mu < m; ++mu) off += 2 * (int64_t)(L + 1 - mu) * kC * (L + 1 - mu) * kC;
  return off;
}
// B matrices of block m: W0 (m = 0), or W1_m and W2_m; the minus sign of the
// complex product is applied by flipping W2's sign bits in registers.
__host__ __device__ constexpr int n_bmat(int m) { return m ? 2 : 1; }
// entries of the fragment-ordered weights (the same count as w_so2)
__host__ __device__ constexpr int64_t wf_entries(int L) { return w1_offset(L, L + 1); }

struct MfmaParams {
  const float* pos;
  const int32_t* row_ptr;
  const int32_t* col;
  const int32_t* gs;      // first target of every group, gs[n_groups] = n_targets
  const uint32_t* xp;     // x repacked as component pairs [n_atoms][pair_off(L+1)][C]
  const float* wrad;      // w_rad in fp32 [K][C]
  const uint16_t* wf;     // w_so2 in MFMA fragment order
  const float* q;
  const float* k;
  float* stat_max;  // [n_targets][H]
  float* stat_inv;  // [n_targets][H]
  float* y;
  const uint16_t* w_logit;  // [K][H] bf16 radial logit bias, or null
  uint32_t xp_bytes;  // extent of xp for its buffer descriptor
  uint32_t w_bytes;   // extent of w_so2
  int32_t n_targets, H, K, p;
  int32_t m_max;  // the per-m maps stop at |m| = m_max (L: every order)
  int32_t n_focus;          // F focus streams of C / F channels (1: one)
  const uint16_t* w_focus;  // [C] bf16 focus score weights (F > 1)
  float cutoff;
  uint32_t flags;
  int32_t periodic;
  float box[3];
};

// Two floats to packed bf16 (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ inline unsigned int pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// a.lo * b.lo + a.hi * b.hi + c (bf16 pairs, fp32 accumulate).
__device__ inline float dot2(unsigned int a, unsigned int b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// a.lo * b.lo + a.hi * b.hi.  Written with the builtin (a move of 0 plus
// the accumulating form), not as inline asm: the compiler cannot see the
// registers an asm statement writes when it inserts the wait states that
// keep a VALU write off the operands and result registers of an MFMA still
// in flight.
__device__ inline float dot2_0(unsigned int a, unsigned int b) { return dot2(a, b, 0.0f); }

// Raw buffer descriptor (gfx9 family: dword3 = 0x00020000).  Loads through
// it take one 32-bit VGPR offset plus a scalar offset and return 0 past
// num_records bytes.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ inline u32x2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

// One gather vector (16 or 8 bytes).
template <int G>
__device__ inline typename XVec<G>::type buffer_load_x(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (G == 4) return buffer_load16(r, voff, soff);
  else return buffer_load8(r, voff, soff);
}

// Radial logit bias of head h for an edge of length rho: sum_k phi_k(rho)
// w_logit[k][h] (0 without the bias).
__device__ inline float logit_bias(const MfmaParams& P, float rho, int h) {
  if (!P.w_logit) return 0.0f;
  const float step = P.cutoff / (float)(P.K - 1);
  const float inv2s2 = 1.0f / (2.0f * step * step);
  float b = 0.0f;
  for (int kk = 0; kk < P.K; ++kk) {
    const float dr = rho - step * (float)kk;
    b += expf(-dr * dr * inv2s2) * bf16_to_float(P.w_logit[kk * P.H + h]);
  }
  return b;
}

// ---------------------------------------------------------------- prologue

// x [n][(L+1)^2][C] bf16 -> xp [n][pair_off(L+1)][C] dwords, dword (l, p, c)
// = x[l^2 + 2p][c] | x[l^2 + 2p + 1][c] << 16 (upper half 0 for p = l),
// four channels per thread;
// w_rad bf16 -> fp32;
// w_so2 -> fragment order: each matrix (W0, then W1_m, W2_m for m = 1..m_max,
// at the same offsets) is cut into 16-row x 32-column blocks, block (row
// tile R, K step s) at (R (KM / 32) + s) KB, and lane (row % 16) + 16
// ((col % 32) / 8) of a block holds its 8 consecutive columns, so one
// 16-byte load per lane reads a whole MFMA B fragment from 1 KB of memory.
template <int L>
__global__ void __launch_bounds__(256) attn_pack_kernel(const uint16_t* __restrict__ x, uint32_t* __restrict__ xp,
                                                        int n_atoms, const uint16_t* __restrict__ w_rad,
                                                        float* __restrict__ wrad, int n_rbf,
                                                        const uint16_t* __restrict__ w_so2,
                                                        uint16_t* __restrict__ wf, int64_t w_entries, int F) {
  constexpr int NC = (L + 1) * (L + 1);
  constexpr int NP = pair_off(L + 1);
  const int64_t n_x = (int64_t)n_atoms * NP * (kC / 4);
  const int64_t n_w = (int64_t)n_rbf * kC;
  // the blocks m <= m_max that w_so2 holds (one stream), or the dense
  // block-diagonal matrices of F streams
  const int64_t n_f = (F == 1 ? w_entries : wf_entries(L)) / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_x + n_w + n_f; i += stride) {
    if (i < n_x) {
      const int c4 = (int)(i % (kC / 4));
      const int pi = (int)((i / (kC / 4)) % NP);
      const int64_t a = i / ((kC / 4) * NP);
      int l = 0;
      while (pair_off(l + 1) <= pi) ++l;
      const int pp = pi - pair_off(l);
      const int comp = l * l + 2 * pp;
      typedef __attribute__((ext_vector_type(4))) unsigned short u16x4;
      const u16x4 lo = *(const u16x4*)(x + (a * NC + comp) * kC + 4 * c4);
      u16x4 hi = {0, 0, 0, 0};
      if (pp < l) hi = *(const u16x4*)(x + (a * NC + comp + 1) * kC + 4 * c4);
      u32x4 o;
      o.x = (uint32_t)lo.x | ((uint32_t)hi.x << 16);
      o.y = (uint32_t)lo.y | ((uint32_t)hi.y << 16);
      o.z = (uint32_t)lo.z | ((uint32_t)hi.z << 16);
      o.w = (uint32_t)lo.w | ((uint32_t)hi.w << 16);
      *(u32x4*)(xp + ((a * NP + pi) * kC + 4 * c4)) = o;
    } else if (i < n_x + n_w) {
      const int64_t w = i - n_x;
      wrad[w] = bf16_to_float(w_rad[w]);
    } else {
      const int64_t g = 8 * (i - n_x - n_w);  // first element of this lane's 16 bytes in wf
      int64_t base = 0;  // first entry of the matrix (the same in wf and in w_so2)
      int mi = 0, KM = (L + 1) * kC;
      while (g >= base + (int64_t)KM * KM) {
        base += (int64_t)KM * KM;
        ++mi;
        KM = (L + 1 - (mi + 1) / 2) * kC;
      }
      const int64_t lg = (g - base) / 8;
      const int lane = (int)(lg % 64);
      const int64_t f = lg / 64;
      const int ks = (int)(f % (KM / 32));
      const int64_t row = 16 * (f / (KM / 32)) + (lane & 15);
      const int col = 32 * ks + 8 * (lane >> 4);
      if (F == 1) {
        *(u32x4*)(wf + g) = *(const u32x4*)(w_so2 + base + row * KM + col);
      } else {
        // F streams: the dense matrix is block-diagonal over the streams,
        // stream s's block being matrix mi of stack s (the same packing
        // over C' = C / F channels, stacks back to back in w_so2)
        const int Cs = kC / F;
        const int co = (int)(row % kC), ci = col % kC;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (co / Cs == ci / Cs) {
          const int st = co / Cs;
          int64_t sbase = 0;  // matrix mi within a stack
          int KMs = (L + 1) * Cs;
          for (int k = 0; k < mi; ++k) {
            sbase += (int64_t)KMs * KMs;
            KMs = (L + 1 - (k + 2) / 2) * Cs;
          }
          const int64_t per = w_entries / F;
          const int64_t rs = (row / kC) * Cs + (co - st * Cs), cs = (col / kC) * Cs + (ci - st * Cs);
          v = *(const u32x4*)(w_so2 + st * per + sbase + rs * KMs + cs);
        }
        *(u32x4*)(wf + g) = v;
      }
    }
  }
}

// ---------------------------------------------------------------- statistics

// One wave per target (4 per block); the neighbours go in batches of 64.
// First each lane takes one neighbour of the batch: its source j and
// envelope u (geometry once per edge).  Then each half-wave takes one
// neighbour at a time (the halves take alternate ones, kStatUnroll in
// flight), with j and u shuffled from the lane that owns the edge: lane c4
// of a half holds channels 4 c4 .. 4 c4 + 3 of q_t and reads the same
// channels of k_j, so one neighbour's k row is one coalesced 512-byte load.
// The d / 4 lanes of a head sum their partial products by xor shuffles
// (d = C / H, a power of two for H <= 16) and keep the head's online
// (max, normaliser) pair over their half's neighbours; the halves are
// combined at the end.
constexpr int kStatUnroll = 4;
__global__ void __launch_bounds__(256) attn_stats_kernel(MfmaParams P, int C) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  if (t >= P.n_targets) return;
  const int half = lane >> 5, c4 = lane & 31;
  const int H = P.H, d = kC / H, gl = d / 4;  // lanes per head
  const int h = c4 / gl;
  const float inv_sqrt_d = 1.0f / sqrtf((float)d);
  const f32x4 qv = *(const f32x4*)(P.q + (int64_t)t * kC + 4 * c4);
  const int e0 = P.row_ptr[t], e1 = P.row_ptr[t + 1];
  float m = -INFINITY, ssum = 0.0f;
  for (int b0 = e0; b0 < e1; b0 += 64) {
    const int nb = min(64, e1 - b0);
    // one edge per lane: source and envelope
    int jl = t;
    float ul = 0.0f, rl = 0.0f;
    if (lane < nb) {
      jl = P.col[b0 + lane];
      const EdgeGeo g = edge_geometry(P.pos, t, jl, P.periodic, P.box, P.cutoff);
      ul = envelope_u(g.s, g.t, P.p);
      rl = g.rho;
    }
    // one edge per half-wave: logits per head and the online softmax (both
    // halves run every iteration, so that the shuffles see all 64 lanes)
    for (int i0 = 0; i0 < nb; i0 += 2 * kStatUnroll) {
      const int i = i0 + half;
      int j[kStatUnroll];
      float u[kStatUnroll], rr[kStatUnroll];
      f32x4 kv[kStatUnroll];
#pragma unroll
      for (int v = 0; v < kStatUnroll; ++v) {
        const int src = min(i + 2 * v, 63);
        j[v] = __shfl(jl, src, 64);
        u[v] = __shfl(ul, src, 64);
        rr[v] = __shfl(rl, src, 64);
      }
#pragma unroll
      for (int v = 0; v < kStatUnroll; ++v) kv[v] = *(const f32x4*)(P.k + (int64_t)j[v] * kC + 4 * c4);
#pragma unroll
      for (int v = 0; v < kStatUnroll; ++v) {
        float z = qv.x * kv[v].x + qv.y * kv[v].y + qv.z * kv[v].z + qv.w * kv[v].w;
        for (int off = 1; off < gl; off <<= 1) z += __shfl_xor(z, off, 64);
        if (i + 2 * v < nb) {
          z = z * inv_sqrt_d + logit_bias(P, rr[v], h);
          if (z > m) {
            ssum = ssum * expf(m - z) + u[v];
            m = z;
          } else {
            ssum += u[v] * expf(z - m);
          }
        }
      }
    }
  }
  // combine the two halves (lanes c4 and c4 + 32 hold the same head)
  const float mo = __shfl_xor(m, 32, 64), so = __shfl_xor(ssum, 32, 64);
  const float M = fmaxf(m, mo);
  const float S = (m == -INFINITY ? 0.0f : ssum * expf(m - M)) + (mo == -INFINITY ? 0.0f : so * expf(mo - M));
  if (half == 0 && c4 % gl == 0) {
    P.stat_max[(int64_t)t * H + h] = M;
    P.stat_inv[(int64_t)t * H + h] = S > 0.0f ? 1.0f / S : 0.0f;
  }
}

// ---------------------------------------------------------------- layout

template <int L>
struct Cfg {
  static constexpr int NC = (L + 1) * (L + 1);
  static constexpr int NP = pair_off(L + 1);   // x pairs per channel
  static constexpr int DPW = dpair_off(L + 1); // Wigner-D pair dwords per edge
  // target accumulator rows (l, slot, m') packed: kSlots l^2 + slot (2l+1) + m' + l
  static constexpr int TROWS = kSlots * NC;
  static constexpr int TT = (TROWS + 15) / 16;  // 16-row MFMA tiles
};

template <int NRI>
struct SmemT {
  int rp[kSlots + 2];   // row_ptr[t_first .. t_first + kSlots]
  int flush_t[kSlots];  // target written out from each slot after this chunk, or -1
  int row_j[kMaxM];
  int row_slot[kMaxM];
  uint16_t rowinfo[NRI];  // accumulator row R -> slot << 8 | component, 0xffff past the rows
  int row_t[kMaxM];       // target of each edge row
  f32x4 row_rv[kMaxM];    // minimum-image edge vector and its length
  float row_u[kMaxM];     // envelope of each edge row
};
// the row table covers the accumulator tiles (at least 112 entries)
template <int L>
using Smem = SmemT<(16 * Cfg<L>::TT > 112 ? 16 * Cfg<L>::TT : 112)>;

// Passes in execution order: blocks m = 1..MM (MM = m_max, L for the base
// layer: the blocks above m_max are not computed), each in groups of at
// most two output degrees (the limit of the register and LDS budgets with
// two sign planes and 64-edge chunks; three with the 32-edge chunks of
// L >= 5), then m = 0 in one pass over all its L + 1 output degrees.  Every
// pass generates, during its last A chunk, the first A chunk of the pass
// after it; ending on m = 0 means a pass never has to produce more sign
// planes than it has itself (an m >= 1 pass writes both planes, m = 0
// reads one).
struct PassInfo {
  int M, LO, ND;
};

__host__ __device__ constexpr PassInfo pass_info(int L, int idx, int MM) {
  int i = 0;
  for (int mm = 1; mm <= MM + 1; ++mm) {
    const int M = mm == MM + 1 ? 0 : mm;
    const int nd = M == 0 ? L + 1 : (L <= 4 ? 2 : 3);
    for (int lo = M; lo <= L; lo += nd) {
      if (i == idx) return PassInfo{M, lo, (L + 1 - lo) < nd ? (L + 1 - lo) : nd};
      ++i;
    }
  }
  return PassInfo{-1, -1, 0};
}

__host__ __device__ constexpr int deg_tiles(int l) {
  return (kSlots * (l + 1) * (l + 1) - 1) / 16 - (kSlots * l * l) / 16 + 1;
}

// A' fragments of pass idx: (degree, tile, K step) for its output degrees.
__host__ __device__ constexpr int frag_count(int L, int idx, int MM) {
  const PassInfo pi = pass_info(L, idx, MM);
  const int rt = chunk_edges(L) / 16;
  const int steps = pi.M == 0 ? rt / 2 : rt;
  int t = 0;
  for (int di = 0; di < pi.ND; ++di) t += deg_tiles(pi.LO + di) * steps;
  return t;
}

// the most A' fragments of any pass (the passes of m_max < L are a subset
// of those of the base layer)
__host__ __device__ constexpr int max_frags(int L) {
  int m = 0;
  for (int i = 0; pass_info(L, i, L).M >= 0; ++i) m = frag_count(L, i, L) > m ? frag_count(L, i, L) : m;
  return m;
}

// A chunks (one degree of one block, 128 channels) of the passes before idx.
__host__ __device__ constexpr int chunks_before(int L, int idx, int MM) {
  int c = 0;
  for (int i = 0; i < idx; ++i) c += L + 1 - pass_info(L, i, MM).M;
  return c;
}

template <int L>
struct Lds {
  static constexpr int M = Geo<L>::M;
  static constexpr size_t kHdr = (sizeof(Smem<L>) + 15) & ~(size_t)15;
  static constexpr size_t kD = kHdr;                                            // u32 [M][DPW]
  static constexpr size_t kG = (kD + 4 * M * Cfg<L>::DPW + 15) & ~(size_t)15;  // f32 [M][kC], swizzled
  static constexpr size_t kW = kG + sizeof(float) * M * kC;                     // f32 [kMaxHeads][M]
  static constexpr size_t kA = kW + sizeof(float) * M * kMaxHeads;              // bf16 [2][2][M][kKC], swizzled
  static constexpr size_t kF = kA + sizeof(uint16_t) * 2 * Geo<L>::ABUF;        // A' fragments u32x4 [][64]
  static constexpr size_t kPhi = kF + sizeof(u32x4) * 64 * max_frags(L);        // f32 [M][kMaxRbf]
  static constexpr size_t kTotal = kPhi + sizeof(float) * M * kMaxRbf;
  // L >= 5, phase A only: D^1, D^4 and D^5 of every edge in fp32, in the
  // A buffers (free until the first A chunk is generated)
  static constexpr size_t kS1 = kA;
  static constexpr size_t kS4 = kS1 + sizeof(float) * M * 9;
  static constexpr size_t kS5 = kS4 + sizeof(float) * M * 81;
  static_assert(L <= 4 || kS5 + sizeof(float) * M * 121 <= kF, "Wigner-D staging fits the A buffers");
};

// 16-byte column groups are XOR-swizzled by row so that both the MFMA
// operand reads (16 rows, one group) and the generator's writes (8 or 4 rows
// x 4 groups per wave) spread over distinct bank groups.
__device__ inline int a_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ inline int a_off(int row, int group) { return row * kKC + 8 * (group ^ a_swz(row)); }
// gate rows: 32 groups of 4 floats, swizzled by row; in K step k the
// generator reads groups 8 k .. 8 k + 7 of each of its rows
__device__ inline int g_swz(int row) { return ((row & 1) << 3) | ((row >> 1) & 1); }
__device__ inline int g_off(int row, int group) { return row * kC + 4 * (group ^ g_swz(row)); }

// Edge er of the chunk: its target t (one of the slots' targets).
template <class SM>
__device__ inline void row_edge(const SM& S, int er, int t_first, int& t) {
  int s = 0;
  while (s + 1 < kSlots && S.rp[s + 1] <= er) ++s;
  t = t_first + s;
}

// D^l rows of one edge as bf16 pairs: dword (l, a, p) at dpair_off(l) +
// a (l+1) + p holds D^l[a][2p] | D^l[a][2p+1] << 16 (upper half 0 for p = l).
template <int l>
__device__ inline void store_dpairs(const float* D, uint32_t* out) {
  constexpr int n = 2 * l + 1;
#pragma unroll
  for (int a = 0; a < n; ++a)
#pragma unroll
    for (int p = 0; p <= l; ++p)
      out[dpair_off(l) + a * (l + 1) + p] = pack_bf16x2(D[a * n + 2 * p], 2 * p + 1 < n ? D[a * n + 2 * p + 1] : 0.0f);
}

// D^0 .. D^min(L, 4) of one edge as pairs, in registers; for L >= 5 also
// D^1 and D^4 in fp32 (s1, s4), from which the higher degrees follow row by
// row (wigner_row).
template <int L>
__device__ inline void wigner_pairs(const float* R, uint32_t* out, float* s1, float* s4) {
  float D1[9];
  wigner_l1(R, D1);
  out[0] = pack_bf16x2(1.0f, 0.0f);
  if constexpr (L >= 1) store_dpairs<1>(D1, out);
  if constexpr (L >= 5) {
#pragma unroll
    for (int q = 0; q < 9; ++q) s1[q] = D1[q];
  }
  if constexpr (L >= 2) {
    float D2[25];
    wigner_step<2>(D1, D1, D2);
    store_dpairs<2>(D2, out);
    if constexpr (L >= 3) {
      float D3[49];
      wigner_step<3>(D1, D2, D3);
      store_dpairs<3>(D3, out);
      if constexpr (L >= 4) {
        float D4[81];
        wigner_step<4>(D1, D3, D4);
        store_dpairs<4>(D4, out);
        if constexpr (L >= 5) {
#pragma unroll
          for (int q = 0; q < 81; ++q) s4[q] = D4[q];
        }
      }
    }
  }
}

// Row a of D^l (l >= 5) of one edge by the same recursion, from D^1 and
// D^{l-1} in fp32: its pairs into the edge's pair block out and, if kNext,
// the row in fp32 into next (D^l, for degree l + 1).
template <int l, int a, bool kNext>
__device__ inline void wigner_row(const float (&D1)[9], const float* Dp, uint32_t* out, float* next) {
  constexpr int n = 2 * l + 1;
  float v[n];
#pragma unroll
  for (int b = 0; b < n; ++b) v[b] = wigner_entry(l, a - l, b - l, D1, Dp);
  if constexpr (kNext) {
#pragma unroll
    for (int b = 0; b < n; ++b) next[a * n + b] = v[b];
  }
#pragma unroll
  for (int p = 0; p <= l; ++p)
    out[dpair_off(l) + a * (l + 1) + p] = pack_bf16x2(v[2 * p], 2 * p + 1 < n ? v[2 * p + 1] : 0.0f);
}

// wigner_row for a row index known only at run time.
template <int l, int A, bool kNext>
__device__ inline void wigner_row_any(int a, const float (&D1)[9], const float* Dp, uint32_t* out, float* next) {
  if constexpr (A < 2 * l + 1) {
    if (a == A) wigner_row<l, A, kNext>(D1, Dp, out, next);
    else wigner_row_any<l, A + 1, kNext>(a, D1, Dp, out, next);
  }
}

// ---------------------------------------------------------------- A operand

// Per-lane state for one edge chunk.  Generator lane: row r0 = tid / GL
// and, in K step k of an A chunk, the GCH channels 32 k + GCH (tid % GL):
// the GL lanes of a row read one 128-byte line of x pairs per load.
struct Ctx {
  uint32_t xoff[kGR];  // byte offset of (j, pair 0, channel GCH (tid % GL)) in xp per row; xp_bytes if no edge
  int r0, c8;
  int head[kNT];       // head of each of this lane's output column tiles
};

// Gathers of generator unit k of an A chunk of degree glp: for every pair
// p < MP and every generator row one 16- or 8-byte load (p > glp reads past
// the buffer: zeros, no memory traffic, so the code has no branch on glp).
template <int L>
__device__ inline void gen_issue(__amdgpu_buffer_rsrc_t xrs, const Ctx& c, uint32_t oob, int glp, int k,
                                 typename XVec<Geo<L>::GCH>::type (&xr)[kGR * Geo<L>::MP]) {
#pragma unroll
  for (int p = 0; p < Geo<L>::MP; ++p) {
    const uint32_t soff = (uint32_t)((pair_off(glp) + p) * kC + 32 * k) * 4u;
#pragma unroll
    for (int u = 0; u < kGR; ++u) xr[kGR * p + u] = buffer_load_x<Geo<L>::GCH>(xrs, p <= glp ? c.xoff[u] : oob, soff);
  }
}

// D pairs of the generator rows for an A chunk (gm, glp): rows glp + gm and
// glp - gm of D^glp, pairs 0..glp.  Past the last row of a degree lie the
// next edge's pairs or, after the last edge, other LDS data, so the pairs
// past glp are not read: with kZero they are set to zero (for gen_finish,
// which sums every pair; their gathers read zeros too); without it they
// repeat pair glp, for the K steps of the main loop, whose dot products
// stop at the unit's degree.  The reads then need no select after them and
// all go out before the first wait.
template <int L, bool kZero = true>
__device__ inline void gen_dpairs(const uint32_t* sD, const Ctx& c, int gm, int glp,
                                  uint32_t (&dp)[kGR][Geo<L>::MP], uint32_t (&dm)[kGR][Geo<L>::MP]) {
  constexpr int DPW = Cfg<L>::DPW;
#pragma unroll
  for (int u = 0; u < kGR; ++u) {
    const uint32_t* d = sD + (c.r0 + Geo<L>::M * u) * DPW + dpair_off(glp);
#pragma unroll
    for (int p = 0; p < Geo<L>::MP; ++p) {
      const int pc = p <= glp ? p : glp;
      const uint32_t vp = d[(glp + gm) * (glp + 1) + pc];
      const uint32_t vm = d[(glp - gm) * (glp + 1) + pc];
      dp[u][p] = !kZero || p <= glp ? vp : 0u;
      dm[u][p] = !kZero || p <= glp ? vm : 0u;
    }
  }
}

// Gates of a generator lane's GCH channels of row r in K step k.
template <int G>
__device__ inline void load_gate(const float* sG, int r, int k, int c8, float (&g)[G]) {
  if constexpr (G == 4) {
    const f32x4 v = *(const f32x4*)(sG + g_off(r, 8 * k + c8));
    g[0] = v.x;
    g[1] = v.y;
    g[2] = v.z;
    g[3] = v.w;
  } else {
    const f32x2 v = *(const f32x2*)(sG + g_off(r, 8 * k + (c8 >> 1)) + 2 * (c8 & 1));
    g[0] = v.x;
    g[1] = v.y;
  }
}

// Round g * v to bf16 and store the lane's GCH channels of row r, K step k.
template <int G>
__device__ inline void store_a(uint16_t* plane, int r, int k, int c8, const float (&v)[G], const float (&g)[G]) {
  if constexpr (G == 4) {
    const int ao = a_off(r, 4 * k + (c8 >> 1)) + 4 * (c8 & 1);
    *(u32x2*)(plane + ao) = u32x2{pack_bf16x2(v[0] * g[0], v[1] * g[1]), pack_bf16x2(v[2] * g[2], v[3] * g[3])};
  } else {
    const int ao = a_off(r, 4 * k + (c8 >> 2)) + 2 * (c8 & 3);
    *(uint32_t*)(plane + ao) = pack_bf16x2(v[0] * g[0], v[1] * g[1]);
  }
}

// Generator unit k: a[r][c] = g_r[c] sum_p dot2(D pair, x pair) for the
// + row and (NS = 2) the - row, rounded to bf16 into K step k of abuf.
template <int L, int NS>
__device__ inline void gen_finish(const float* sG, const Ctx& c, int k,
                                  const typename XVec<Geo<L>::GCH>::type (&xr)[kGR * Geo<L>::MP],
                                  const uint32_t (&dp)[kGR][Geo<L>::MP], const uint32_t (&dm)[kGR][Geo<L>::MP],
                                  uint16_t* abuf) {
  constexpr int G = Geo<L>::GCH;
#pragma unroll
  for (int u = 0; u < kGR; ++u) {
    const int r = c.r0 + Geo<L>::M * u;
    float ap[G], am[G];
#pragma unroll
    for (int q = 0; q < G; ++q) ap[q] = am[q] = 0.0f;
#pragma unroll
    for (int p = 0; p < Geo<L>::MP; ++p) {
      const typename XVec<G>::type v = xr[kGR * p + u];
#pragma unroll
      for (int q = 0; q < G; ++q) ap[q] = dot2(dp[u][p], v[q], ap[q]);
      if constexpr (NS > 1) {
#pragma unroll
        for (int q = 0; q < G; ++q) am[q] = dot2(dm[u][p], v[q], am[q]);
      }
    }
    float g[G];
    load_gate<G>(sG, r, k, c.c8, g);
    store_a<G>(abuf, r, k, c.c8, ap, g);
    if constexpr (NS > 1) store_a<G>(abuf + Geo<L>::APLANE, r, k, c.c8, am, g);
  }
}

// ---------------------------------------------------------------- main GEMM

// B fragments of one K step of pass (M, LO, ND): for output degree LO + di,
// matrix s (W0 / W1, then W2), column tile nt of this wave: the 1 KB block
// (row tile, K step) of the fragment-ordered weights.  The lane and tile
// part of the address is fixed for the pass; the step part (1 KB per step)
// is the scalar offset.
template <int L, int M>
__device__ constexpr uint32_t bmat_byte(int s) {
  constexpr int KM = (L + 1 - M) * kC;
  constexpr uint32_t w1_byte = (uint32_t)(M == 0 ? 0 : w1_offset(L, M)) * 2u;
  return s == 0 ? w1_byte : w1_byte + (uint32_t)(KM * KM) * 2u;
}

template <int L, int M, int LO, int ND>
__device__ inline void load_b(__amdgpu_buffer_rsrc_t wrs, const uint32_t (&boff)[ND][kNT], int step,
                              u32x4 (&b)[ND][n_bmat(M)][kNT]) {
  const uint32_t sb = 1024u * (uint32_t)step;
#pragma unroll
  for (int di = 0; di < ND; ++di)
#pragma unroll
    for (int sm = 0; sm < n_bmat(M); ++sm)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) b[di][sm][nt] = buffer_load16(wrs, boff[di][nt], bmat_byte<L, M>(sm) + sb);
}

template <int L, int M, int LO, int ND>
__device__ inline void b_offsets(uint32_t (&boff)[ND][kNT]) {
  constexpr int KM = (L + 1 - M) * kC;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int di = 0; di < ND; ++di)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
      boff[di][nt] = 16u * lane + (uint32_t)(((LO + di - M) * 8 + kNT * wave + nt) * (KM / 32)) * 1024u;
}

// One K step with its generator unit.  The loads of the next step are
// spread over the first two thirds of the step's F MFMAs; the generator's D
// dot products follow the last MFMA as one block, then the unit's gate,
// rounding and LDS store.
template <int L, int ND, int NS>
struct StepState {
  typedef typename XVec<Geo<L>::GCH>::type XV;
  static constexpr int RT = Geo<L>::RT, MP = Geo<L>::MP, G = Geo<L>::GCH;
  const u32x4* ap;                      // [RT] + plane fragments
  const u32x4* am;                      // [RT] - plane fragments
  const u32x4 (&b)[ND][n_bmat(NS - 1)][kNT];  // W0, or W1 and W2
  f32x4 (&acc)[ND][NS][kNT][RT];
  const XV (&xr)[kGR * MP];
  const uint32_t (&dp)[kGR][MP];
  const uint32_t (&dm)[kGR][MP];
  float (&vp)[kGR][G];
  float (&vm)[kGR][G];
  // loads for the next K step, spread over the MFMAs of this one
  u32x4 (&bn)[ND][n_bmat(NS - 1)][kNT];  // B fragments of the next step
  __amdgpu_buffer_rsrc_t wrs;
  const uint32_t (&boff)[ND][kNT];
  uint32_t wsoff[2];                    // scalar offsets of the next step's W0 / W1 and W2 blocks
  XV (&xn)[kGR * MP];                   // gathers of the next generator unit
  __amdgpu_buffer_rsrc_t xrs;
  uint32_t xoff[kGR];                   // per row; past the end for pairs beyond the unit's degree
  uint32_t xsoff;                       // scalar offset of the unit's pair 0
  int glp;                              // degree of the next unit's chunk
  uint32_t oob;
  int dglp;                             // degree of this step's unit: pairs 0..dglp are nonzero
};

// Load j of the next-step loads: first the B fragments, then the gathers.
template <int L, int ND, int NS, int J>
__device__ __attribute__((always_inline)) inline void step_load(StepState<L, ND, NS>& st) {
  constexpr int NBM = n_bmat(NS - 1);
  constexpr int NB = ND * NBM * kNT;
  if constexpr (J < NB) {
    constexpr int di = J / (NBM * kNT), sm = (J / kNT) % NBM, nt = J % kNT;
    st.bn[di][sm][nt] = buffer_load16(st.wrs, st.boff[di][nt], st.wsoff[sm]);
  } else {
    constexpr int g = J - NB, p = g / kGR, u = g % kGR;
    if constexpr (L >= 5) {
      // pairs past the next unit's degree are not loaded (their dot products
      // are skipped, so the registers may keep stale values); measured faster
      // at L = 6, while at L <= 4 the branches cost more registers than the
      // loads they save
      if (p == 0 || p <= st.glp)
        st.xn[g] = buffer_load_x<Geo<L>::GCH>(st.xrs, st.xoff[u], st.xsoff + (uint32_t)p * (kC * 4));
    } else {
      st.xn[g] = buffer_load_x<Geo<L>::GCH>(st.xrs, p <= st.glp ? st.xoff[u] : st.oob,
                                            st.xsoff + (uint32_t)p * (kC * 4));
    }
  }
}

template <int L, int ND, int NS, int I>
__device__ __attribute__((always_inline)) inline void step_mfma(StepState<L, ND, NS>& st) {
  constexpr int PR = ND * kNT * NS * NS;  // MFMAs per row tile
  constexpr int rt = I / PR, j = I % PR;
  if constexpr (NS == 1) {
    constexpr int di = j / kNT, nt = j % kNT;
    st.acc[di][0][nt][rt] = mfma(as_bf16x8(st.ap[rt]), as_bf16x8(st.b[di][0][nt]), st.acc[di][0][nt][rt]);
  } else {
    constexpr int ph = j / (2 * ND * kNT), jj = j % (2 * ND * kNT);
    constexpr int di = jj / (2 * kNT), nt = (jj / 2) % kNT, mt = jj % 2;
    if constexpr (ph == 0)
      st.acc[di][mt][nt][rt] = mfma(as_bf16x8(st.ap[rt]), as_bf16x8(st.b[di][mt][nt]), st.acc[di][mt][nt][rt]);
    else if constexpr (mt == 0)
      st.acc[di][0][nt][rt] =
          mfma(as_bf16x8(st.am[rt]),
               as_bf16x8(st.b[di][1][nt] ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}),
               st.acc[di][0][nt][rt]);
    else
      st.acc[di][1][nt][rt] = mfma(as_bf16x8(st.am[rt]), as_bf16x8(st.b[di][0][nt]), st.acc[di][1][nt][rt]);
  }
}

template <int L, int ND, int NS, int D0, int D1>
__device__ __attribute__((always_inline)) inline void step_dots(StepState<L, ND, NS>& st) {
  constexpr int G = Geo<L>::GCH;
  if constexpr (D0 < D1) {
    constexpr int p = D0 / (G * kGR * NS), r = D0 % (G * kGR * NS);
    constexpr int u = r / (G * NS), q = (r / NS) % G, sg = r % NS;
    const typename XVec<G>::type v = st.xr[kGR * p + u];
    const uint32_t xv = v[q];
    // pair 0 starts the sum: its accumulator input is the constant 0
    if constexpr (p == 0 && sg == 0) st.vp[u][q] = dot2_0(st.dp[u][p], xv);
    else if constexpr (p == 0) st.vm[u][q] = dot2_0(st.dm[u][p], xv);
    else if constexpr (sg == 0) st.vp[u][q] = dot2(st.dp[u][p], xv, st.vp[u][q]);
    else st.vm[u][q] = dot2(st.dm[u][p], xv, st.vm[u][q]);
    step_dots<L, ND, NS, D0 + 1, D1>(st);
  }
}

// The dot products of pairs P, P + 1, ... up to the unit's degree: the pairs
// past it hold zeros on both sides, so they are skipped (a wave-uniform
// branch per pair; the unit's degree is the same for every lane).
template <int L, int ND, int NS, int P>
__device__ __attribute__((always_inline)) inline void step_dots_pairs(StepState<L, ND, NS>& st) {
  constexpr int PD = Geo<L>::GCH * kGR * NS;  // dot products per pair
  if constexpr (P < Geo<L>::MP) {
    if (P == 0 || P <= st.dglp) {
      step_dots<L, ND, NS, P * PD, (P + 1) * PD>(st);
      step_dots_pairs<L, ND, NS, P + 1>(st);
    }
  }
}

template <int L, int ND, int NS, int I>
__device__ __attribute__((always_inline)) inline void step_seq(StepState<L, ND, NS>& st) {
  constexpr int F = ND * kNT * NS * NS * Geo<L>::RT;
  constexpr int NL = ND * n_bmat(NS - 1) * kNT + kGR * Geo<L>::MP;  // loads of the next step
  constexpr int SP = (2 * F / 3) / NL > 0 ? (2 * F / 3) / NL : 1;
  if constexpr (I < F) {
    step_mfma<L, ND, NS, I>(st);
    if constexpr (I % SP == 0 && I / SP < NL) step_load<L, ND, NS, I / SP>(st);
    if constexpr (I == F - 1) {
      // the dot products go after the step's last MFMA, as one block: on
      // gfx950 v_dot2_f32_bf16 does not overlap with MFMAs, and interleaving
      // the two measured about 10 % slower than issuing them in sequence
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      step_dots_pairs<L, ND, NS, 0>(st);
    }
    step_seq<L, ND, NS, I + 1>(st);
  } else if constexpr (I / SP < NL) {
    // more loads than MFMA slots: issue the rest
    step_load<L, ND, NS, I / SP>(st);
    step_seq<L, ND, NS, I + SP>(st);
  }
}

// K step k of an A chunk: MFMAs on the current chunk (abuf) with B
// fragments b, interleaved with generator unit k of the next chunk from the
// gathers xr (written into anext) and with the loads of the next K step:
// its B fragments (step nstep) into bn and the gathers of the next
// generator unit (slice nk of a chunk of degree nglp) into xn.
template <int L, int M, int LO, int ND>
__device__ inline void fused_step(const uint16_t* abuf, int k, int dglp, const u32x4 (&b)[ND][n_bmat(M)][kNT],
                                  f32x4 (&acc)[ND][M ? 2 : 1][kNT][Geo<L>::RT], const float* sG, const Ctx& c,
                                  const typename XVec<Geo<L>::GCH>::type (&xr)[kGR * Geo<L>::MP],
                                  const uint32_t (&dp)[kGR][Geo<L>::MP], const uint32_t (&dm)[kGR][Geo<L>::MP],
                                  uint16_t* anext, u32x4 (&bn)[ND][n_bmat(M)][kNT], __amdgpu_buffer_rsrc_t wrs,
                                  const uint32_t (&boff)[ND][kNT], int nstep,
                                  typename XVec<Geo<L>::GCH>::type (&xn)[kGR * Geo<L>::MP],
                                  __amdgpu_buffer_rsrc_t xrs, int nglp, int nk, uint32_t oob) {
  constexpr int NS = M ? 2 : 1;
  constexpr int RT = Geo<L>::RT, G = Geo<L>::GCH;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int grp = 4 * k + (lane >> 4);
  u32x4 ap[RT], am[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int o = a_off(16 * rt + l16, grp);
    ap[rt] = *(const u32x4*)(abuf + o);
    if constexpr (NS > 1) am[rt] = *(const u32x4*)(abuf + Geo<L>::APLANE + o);
  }
  float vp[kGR][G], vm[kGR][G];  // every entry is first written by its pair-0 dot product
  // gates of the unit's rows and channels, read before the MFMAs so that the
  // LDS latency is hidden behind them
  float gate[kGR][G];
#pragma unroll
  for (int u = 0; u < kGR; ++u) load_gate<G>(sG, c.r0 + Geo<L>::M * u, k, c.c8, gate[u]);
  const uint32_t sb = 1024u * (uint32_t)nstep;
  uint32_t xo[kGR];
#pragma unroll
  for (int u = 0; u < kGR; ++u) xo[u] = c.xoff[u];
  StepState<L, ND, NS> st{ap, am, b, acc, xr, dp, dm, vp, vm,
                          bn, wrs, boff, {bmat_byte<L, M>(0) + sb, bmat_byte<L, M>(1) + sb},
                          xn, xrs, {}, (uint32_t)(pair_off(nglp) * kC + 32 * nk) * 4u, nglp, oob, dglp};
#pragma unroll
  for (int u = 0; u < kGR; ++u) st.xoff[u] = xo[u];
  // the MFMA part of the step runs at raised wave priority, the dot products
  // and LDS stores after it at normal priority (measured about 2 % faster)
  __builtin_amdgcn_s_setprio(1);
  step_seq<L, ND, NS, 0>(st);
#pragma unroll
  for (int u = 0; u < kGR; ++u) {
    const int r = c.r0 + Geo<L>::M * u;
    store_a<G>(anext, r, k, c.c8, vp[u], gate[u]);
    if constexpr (NS > 1) store_a<G>(anext + Geo<L>::APLANE, r, k, c.c8, vm[u], gate[u]);
  }
}

// ---------------------------------------------------------------- rotate back

// Rotate back and sum over neighbours for output degree l of block m:
//   T[l] += A'(D, slots) x B'(w * yt).
// yt[s][nt][rt] is the main GEMM accumulator of this degree (s = 0: +m or
// m = 0, s = 1: -m), lane rows 4 (lane/16) + i of row tile rt, column lane %
// 16 of column tile nt.  B' is yt scaled by the lane's head weight and
// rounded to bf16, packed so that K index 8 g + jj of lane group g is
//   m > 0:  edge 16 st + 4 g + (jj & 3), sign + for jj < 4, - otherwise
//   m = 0:  edge 16 (2 st + jj / 4) + 4 g + (jj & 3);
// A' row R of the accumulator (R = kSlots l^2 + slot (2l+1) + m' + l) holds
// D^l_e[l +- m][m' + l] in the same K order when edge e belongs to that
// slot's target, 0 otherwise (and 0 on rows of other degrees).  A' does not
// depend on the output channels, so the workgroup builds it once per pass
// into LDS (aprime_build) and every wave reads it from there.  The target
// accumulators T stay in registers, in the MFMA C layout.

// A' fragments of pass PI, in the order (degree, tile, K step), 64 lanes x
// 16 bytes each.  Wave w builds fragments w, w + 4, ...; the fragment decode
// is wave-uniform.
template <int L, int MM, int PI>
__device__ inline void aprime_build(char* smem, u32x4* frag) {
  constexpr PassInfo pi = pass_info(L, PI, MM);
  constexpr int M = pi.M, LO = pi.LO;
  constexpr int STEPS = M == 0 ? Geo<L>::RT / 2 : Geo<L>::RT;
  constexpr int TOTAL = frag_count(L, PI, MM);
  const Smem<L>& S = *(const Smem<L>*)smem;
  const uint32_t* sD = (const uint32_t*)(smem + Lds<L>::kD);
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int f = wave; f < TOTAL; f += kWaves) {
    int ff = f, l = LO;
    while (ff >= deg_tiles(l) * STEPS) {
      ff -= deg_tiles(l) * STEPS;
      ++l;
    }
    const int ot = (kSlots * l * l) / 16 + ff / STEPS;
    const int st = ff % STEPS;
    const int n = 2 * l + 1;
    const int rr = 16 * ot + (lane & 15) - kSlots * l * l;
    const bool mine = rr >= 0 && rr < kSlots * n;
    const int oslot = mine ? (int)(((float)rr + 0.5f) * (1.0f / (float)n)) : -1;
    const int omp = mine ? rr - oslot * n : 0;
    const uint32_t* dl = sD + dpair_off(l) + (omp >> 1);
    const int sh = (omp & 1) * 16;
    unsigned int hv[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      int r, srow;
      if constexpr (M > 0) {
        r = 16 * st + 4 * g4 + (jj & 3);
        srow = (jj < 4) ? (l + M) : (l - M);
      } else {
        r = 16 * (2 * st + (jj >> 2)) + 4 * g4 + (jj & 3);
        srow = l;
      }
      const uint32_t w = dl[r * Cfg<L>::DPW + srow * (l + 1)];
      hv[jj] = S.row_slot[r] == oslot ? (w >> sh) & 0xffffu : 0u;
    }
    u32x4 a;
    a.x = hv[0] | (hv[1] << 16);
    a.y = hv[2] | (hv[3] << 16);
    a.z = hv[4] | (hv[5] << 16);
    a.w = hv[6] | (hv[7] << 16);
    frag[f * 64 + lane] = a;
  }
}

template <int L, int NS, int l>
__device__ inline void rot_back(char* smem, const Ctx& c, const f32x4 (&yt)[NS][kNT][Geo<L>::RT], const u32x4* frag,
                                f32x4 (&T)[Cfg<L>::TT][kNT]) {
  constexpr int RT = Geo<L>::RT;
  const float* sW = (const float*)(smem + Lds<L>::kW);
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4;
  constexpr bool M0 = NS == 1;
  constexpr int kSteps = M0 ? RT / 2 : RT;
  constexpr int ot0 = (kSlots * l * l) / 16;
  u32x4 bq[kNT][RT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      // weights of this lane's 4 edge rows for the head of column tile nt
      const f32x4 wv = *(const f32x4*)(sW + c.head[nt] * Geo<L>::M + 16 * rt + 4 * g4);
      const float w4[4] = {wv.x, wv.y, wv.z, wv.w};
      if constexpr (!M0) {
        const f32x4 yp = yt[0][nt][rt], ym = yt[NS - 1][nt][rt];
        bq[nt][rt].x = pack_bf16x2(yp[0] * w4[0], yp[1] * w4[1]);
        bq[nt][rt].y = pack_bf16x2(yp[2] * w4[2], yp[3] * w4[3]);
        bq[nt][rt].z = pack_bf16x2(ym[0] * w4[0], ym[1] * w4[1]);
        bq[nt][rt].w = pack_bf16x2(ym[2] * w4[2], ym[3] * w4[3]);
      } else {
        const f32x4 y0 = yt[0][nt][rt];
        const unsigned int lo01 = pack_bf16x2(y0[0] * w4[0], y0[1] * w4[1]);
        const unsigned int lo23 = pack_bf16x2(y0[2] * w4[2], y0[3] * w4[3]);
        if ((rt & 1) == 0) {
          bq[nt][rt].x = lo01;
          bq[nt][rt].y = lo23;
        } else {
          bq[nt][rt - 1].z = lo01;
          bq[nt][rt - 1].w = lo23;
        }
      }
    }
#pragma unroll
  for (int q = 0; q < deg_tiles(l); ++q)
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const u32x4 a = frag[(q * kSteps + st) * 64 + lane];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        T[ot0 + q][nt] = mfma(as_bf16x8(a), as_bf16x8(bq[nt][M0 ? 2 * st : st]), T[ot0 + q][nt]);
    }
}

template <int L, int M, int LO, int DI, int ND>
__device__ inline void rot_back_all(char* smem, const Ctx& c, const f32x4 (&acc)[ND][M ? 2 : 1][kNT][Geo<L>::RT],
                                    const u32x4* frag, f32x4 (&T)[Cfg<L>::TT][kNT]) {
  constexpr int STEPS = M == 0 ? Geo<L>::RT / 2 : Geo<L>::RT;
  rot_back<L, M ? 2 : 1, LO + DI>(smem, c, acc[DI], frag, T);
  if constexpr (DI + 1 < ND)
    rot_back_all<L, M, LO, DI + 1, ND>(smem, c, acc, frag + deg_tiles(LO + DI) * STEPS * 64, T);
}

// ---------------------------------------------------------------- passes

// Generation target of A chunk q of pass PI (the chunk written while chunk
// q is multiplied): the next degree of the same block, else the first
// chunk of the next pass; after the last pass a dummy (degree 0 of m = 0)
// whose result nobody reads.
template <int L, int MM, int PI>
__device__ inline void gen_target(int q, int& gm, int& glp) {
  constexpr PassInfo pi = pass_info(L, PI, MM), pn = pass_info(L, PI + 1, MM);
  constexpr int NCH = L + 1 - pi.M;
  if (q + 1 < NCH) {
    gm = pi.M;
    glp = pi.M + q + 1;
  } else {
    gm = pn.M >= 0 ? pn.M : 0;
    glp = pn.M >= 0 ? pn.M : 0;
  }
}

// One pass: block M, output degrees LO .. LO+ND-1.  On entry the B fragments
// of K step 0 are in flight in ring[0] and the gathers of generator unit 0
// of chunk 0's target in xa; A chunk 0 is in LDS buffer chunks_before(L, PI, MM) & 1
// once every wave has reached the first barrier.
//
// K step s = 4 q + k multiplies A chunk q (degree M + q, channels 32 k ..
// 32 k + 31) with ring[s & 1] while the B fragments of step s + 1 load into
// ring[(s + 1) & 1]; its VALU work, generator unit k of the chunk after q
// (slice k of the other buffer), uses gathers issued one step earlier and is
// interleaved with the MFMAs.  The loop body is two K steps; one barrier
// per A chunk.
template <int L, int MM, int PI>
__device__ __attribute__((always_inline)) inline void run_pass(const MfmaParams& P, char* smem, const Ctx& c,
                                                               f32x4 (&T)[Cfg<L>::TT][kNT],
                                                               u32x4 (&ring)[2][pass_info(L, PI, MM).ND]
                                                                            [n_bmat(pass_info(L, PI, MM).M)][kNT],
                                                               typename XVec<Geo<L>::GCH>::type (&xa)[kGR * Geo<L>::MP],
                                                               typename XVec<Geo<L>::GCH>::type (&xb)[kGR * Geo<L>::MP]) {
  constexpr PassInfo pi = pass_info(L, PI, MM), pn = pass_info(L, PI + 1, MM);
  constexpr int M = pi.M, LO = pi.LO, ND = pi.ND, NS = M ? 2 : 1;
  constexpr int RT = Geo<L>::RT, MP = Geo<L>::MP;
  constexpr int NCH = L + 1 - M, NSTEP = 4 * NCH;
  constexpr int PAR = chunks_before(L, PI, MM) & 1;
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(P.wf, P.w_bytes);
  const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(P.xp, P.xp_bytes);
  const uint32_t* sD = (const uint32_t*)(smem + Lds<L>::kD);
  const float* sG = (const float*)(smem + Lds<L>::kG);
  uint16_t* abase = (uint16_t*)(smem + Lds<L>::kA);
  u32x4* frag = (u32x4*)(smem + Lds<L>::kF);
  const uint32_t oob = P.xp_bytes;

  uint32_t boff[ND][kNT];
  b_offsets<L, M, LO, ND>(boff);

  __syncthreads();  // chunk 0 written; every wave is done with the previous A'
  aprime_build<L, MM, PI>(smem, frag);

  f32x4 acc[ND][NS][kNT][RT];
#pragma unroll
  for (int a = 0; a < ND; ++a)
#pragma unroll
    for (int b = 0; b < NS; ++b)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[a][b][nt][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  uint32_t dp[kGR][MP], dm[kGR][MP];
  int glp = 0;
#pragma nounroll
  for (int s = 0; s < NSTEP; s += 2) {
    const int q = s >> 2;
    const int k = s & 3;  // 0 or 2
    if (k == 0) {
      int gm;
      gen_target<L, MM, PI>(q, gm, glp);
      gen_dpairs<L, false>(sD, c, gm, glp, dp, dm);
    }
    // degree of the chunk whose generator unit 0 is gathered in step s + 1
    int glp2 = glp;
    if (k == 2) {
      // at the pass's last A chunk, step s + 2 is the next pass's first
      // step, whose generator unit 0 belongs to that pass's chunk 1 target
      int gm2;
      if (q + 1 < NCH) {
        gen_target<L, MM, PI>(q + 1, gm2, glp2);
      } else {
        if constexpr (pn.M >= 0) gen_target<L, MM, PI + 1>(0, gm2, glp2);
        else gen_target<L, MM, PI>(q, gm2, glp2);
      }
    }
    const uint16_t* acur = abase + ((PAR + q) & 1) * Geo<L>::ABUF;
    uint16_t* anext = abase + ((PAR + q + 1) & 1) * Geo<L>::ABUF;
    // K step s: unit k from xa; loads B of step s + 1 and the gathers of unit k + 1
    fused_step<L, M, LO, ND>(acur, k, glp, ring[0], acc, sG, c, xa, dp, dm, anext, ring[1], wrs, boff, s + 1, xb, xrs,
                             glp, k + 1, oob);
    // K step s + 1: unit k + 1 from xb; loads B of step s + 2 and the gathers of the next unit
    fused_step<L, M, LO, ND>(acur, k + 1, glp, ring[1], acc, sG, c, xb, dp, dm, anext, ring[0], wrs, boff,
                             min(s + 2, NSTEP - 1), xa, xrs, glp2, (k + 2) & 3, oob);
    if (k == 2) __syncthreads();  // chunk q + 1 written, chunk q read by every wave
  }

  if constexpr (pn.M >= 0) {
    constexpr int NDn = pn.ND;
    u32x4 nring[2][NDn][n_bmat(pn.M)][kNT];
    uint32_t nboff[NDn][kNT];
    b_offsets<L, pn.M, pn.LO, NDn>(nboff);
    load_b<L, pn.M, pn.LO, NDn>(wrs, nboff, 0, nring[0]);
    // the gathers of the next pass's first generator unit are in xa (issued
    // by the last K step)
    rot_back_all<L, M, LO, 0, ND>(smem, c, acc, frag, T);
    run_pass<L, MM, PI + 1>(P, smem, c, T, nring, xa, xb);
  } else {
    rot_back_all<L, M, LO, 0, ND>(smem, c, acc, frag, T);
  }
}

// ---------------------------------------------------------------- focus streams

// Cross-focus softmax of F streams (L <= 4; F divides the head count, so
// every head lies in one stream): per edge, score_f = sum over the
// stream's channels c of w_focus[c] yt[(0,0), c], the stream's invariant
// l = 0 output of the m = 0 map in the edge frame, and pi_f = softmax_f;
// pi then scales the softmax weights of the stream's heads in LDS, so the
// rotate-back of every pass applies it.  yt[(0,0), .] is the m = 0 map's
// output degree 0: a GEMM over the chunk's m = 0 A chunks (degrees 0..L,
// generated here one after another into the two A buffers) with W0's
// degree-0 rows, on the matrix cores; the per-wave partial scores (16
// channels each) meet in the A' fragment area, free before the first pass.
template <int L, int F>
__device__ inline void focus_weights(const MfmaParams& P, char* smem, const Ctx& c, int nrows) {
  static_assert(Geo<L>::M == 64, "64-edge chunks (L <= 4)");
  constexpr int RT = Geo<L>::RT, MP = Geo<L>::MP;
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(P.wf, P.w_bytes);
  const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(P.xp, P.xp_bytes);
  const uint32_t* sD = (const uint32_t*)(smem + Lds<L>::kD);
  const float* sG = (const float*)(smem + Lds<L>::kG);
  float* sW = (float*)(smem + Lds<L>::kW);
  uint16_t* abase = (uint16_t*)(smem + Lds<L>::kA);
  float* sScore = (float*)(smem + Lds<L>::kF);  // [kWaves][M]
  const uint32_t oob = P.xp_bytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  uint32_t boff[1][kNT];
  b_offsets<L, 0, 0, 1>(boff);
  f32x4 acc[kNT][RT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[nt][rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  typename XVec<Geo<L>::GCH>::type xa[kGR * MP], xb[kGR * MP];
  for (int lp = 0; lp <= L; ++lp) {
    uint16_t* ab = abase + (lp & 1) * Geo<L>::ABUF;
    // W0's degree-0 rows for the 4 K steps of input degree lp
    u32x4 b[4][1][1][kNT];
#pragma unroll
    for (int k = 0; k < 4; ++k) load_b<L, 0, 0, 1>(wrs, boff, 4 * lp + k, b[k]);
    // the m = 0 A chunk of degree lp (one plane), 4 generator units
    uint32_t dp[kGR][MP], dm[kGR][MP];
    gen_dpairs<L>(sD, c, 0, lp, dp, dm);
    gen_issue<L>(xrs, c, oob, lp, 0, xa);
    gen_issue<L>(xrs, c, oob, lp, 1, xb);
    gen_finish<L, 1>(sG, c, 0, xa, dp, dm, ab);
    gen_issue<L>(xrs, c, oob, lp, 2, xa);
    gen_finish<L, 1>(sG, c, 1, xb, dp, dm, ab);
    gen_issue<L>(xrs, c, oob, lp, 3, xb);
    gen_finish<L, 1>(sG, c, 2, xa, dp, dm, ab);
    gen_finish<L, 1>(sG, c, 3, xb, dp, dm, ab);
    // every wave wrote its part; every wave is done with the chunk before
    // the previous one in this buffer
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int grp = 4 * k + g4;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const u32x4 av = *(const u32x4*)(ab + a_off(16 * rt + l16, grp));
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[nt][rt] = mfma(as_bf16x8(av), as_bf16x8(b[k][0][0][nt]), acc[nt][rt]);
      }
    }
  }
  // partial scores of this wave's 16 channels: lane (g4, l16) holds rows
  // 16 rt + 4 g4 + i of column l16; sum the 16 columns of each row
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const float wfc = bf16_to_float(P.w_focus[16 * kNT * wave + 16 * nt + l16]);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += wfc * acc[nt][rt][i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v[i] += __shfl_xor(v[i], o, 64);
    }
    if (l16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sScore[wave * Geo<L>::M + 16 * rt + 4 * g4 + i] = v[i];
    }
  }
  __syncthreads();
  // one thread per edge row: the streams' scores, their softmax, and the
  // stream factor on the weights of the stream's heads
  constexpr int WPS = kWaves / F;  // waves (16 channels each) per stream
  static_assert(kWaves % F == 0, "whole waves per stream");
  if (threadIdx.x < Geo<L>::M) {
    const int r = threadIdx.x;
    float sc[F];
    float mx = -INFINITY;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < WPS; ++w) t += sScore[(f * WPS + w) * Geo<L>::M + r];
      sc[f] = t;
      mx = fmaxf(mx, t);
    }
    float den = 0.0f;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      sc[f] = expf(sc[f] - mx);
      den += sc[f];
    }
    const float inv = 1.0f / den;
    const int hps = P.H / F;  // heads per stream
    if (r < nrows)
      for (int h = 0; h < P.H; ++h) sW[h * Geo<L>::M + r] *= sc[h / hps] * inv;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- flush

// Accumulator row R = kSlots l^2 + slot (2l+1) + comp - l^2 as slot << 8 |
// comp (0xffff for the padding rows of the last tile).
__device__ inline uint16_t row_info(int R, int TROWS) {
  if (R >= TROWS) return 0xffff;
  int l = 0;
  while (kSlots * (l + 1) * (l + 1) <= R) ++l;
  const int rr = R - kSlots * l * l, n = 2 * l + 1;
  return (uint16_t)(((rr / n) << 8) | (l * l + rr % n));
}

// Write every slot whose target finished in this chunk to y and clear it.
// T[ot][nt] entry i of lane (g, l16) is accumulator row R = 16 ot + 4 g + i,
// column 32 wave + 16 nt + l16.  Straight-line code: each entry looks its
// row up in the row table and its slot's target in flush_t, and lanes with
// nothing to write store past the end of a buffer descriptor that covers
// the chunk's (at most kSlots) target rows of y.
template <int L>
__device__ inline void flush_slots(const MfmaParams& P, const Smem<L>& S, int t_first, f32x4 (&T)[Cfg<L>::TT][kNT]) {
  constexpr int NC = Cfg<L>::NC;
  constexpr uint32_t kRow = NC * kC * 4;  // bytes of one target row of y
  if (S.flush_t[0] < 0 && S.flush_t[1] < 0 && S.flush_t[2] < 0 && S.flush_t[3] < 0) return;
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4;
  const uint32_t colb = 4u * (uint32_t)(16 * kNT * (threadIdx.x >> 6) + (lane & 15));
  const int nt_rows = min(kSlots, P.n_targets - t_first);
  const __amdgpu_buffer_rsrc_t yrs = buffer_rsrc(P.y + (int64_t)t_first * NC * kC, (uint32_t)nt_rows * kRow);
  const uint32_t oob = (uint32_t)kSlots * kRow;
#pragma unroll
  for (int ot = 0; ot < Cfg<L>::TT; ++ot)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int info = S.rowinfo[16 * ot + 4 * g4 + i];
      const int t = S.flush_t[(info >> 8) & (kSlots - 1)];
      const bool out = info != 0xffff && t >= 0;
      const uint32_t off = out ? (uint32_t)(t - t_first) * kRow + (uint32_t)(info & 0xff) * (kC * 4) + colb : oob;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const float v = T[ot][nt][i];
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), yrs, (int)(off + 64u * nt), 0, 0);
        T[ot][nt][i] = out ? 0.0f : v;
      }
    }
}

// ---------------------------------------------------------------- kernel

// Groups of XCD x: the contiguous range [xcd_first(x), xcd_first(x + 1)).
__host__ __device__ inline int xcd_first(int x, int n_groups) {
  const int per = n_groups / 8, rem = n_groups % 8;
  return x * per + (x < rem ? x : rem);
}

// Work of target t in 1/64 of a chunk, an additive estimate of the fused
// kernel's greedy chunking (at most CM edges and kSlots targets per
// chunk): a target takes d / CM chunks, and at least 1 / kSlots of one.
template <int CM>
__device__ inline int64_t target_work(int d) {
  const int64_t w = (int64_t)d * (64 / CM);
  return w > 64 / kSlots ? w : 64 / kSlots;
}

// Run estimate of the fused kernel's schedule (one run of consecutive
// targets per compute unit), one workgroup of 1024 threads.  With W the
// total work and wsum[t] the work of targets 0..t-1, run g of n_groups
// starts at the first target t with wsum[t] >= goal_g = floor(g W /
// n_groups), and run n_groups at n_targets.  Runs are written from the
// prefix sums without a search: the number of runs whose goal is at most X
// is runs_upto(X) = min(n_groups, ceil((X + 1) n_groups / W)), so target i,
// with wsum[i] = a and wsum[i + 1] = b, starts runs [runs_upto(a),
// runs_upto(b)) at i + 1, and run 0 starts at 0.  In the exact mode the row
// offsets are staged in LDS and all targets form one span (kExactItems per
// thread); otherwise a first pass sums W and a second scans the targets in
// spans of kSchedItems per thread, walking the run index along them.  With
// one run per compute unit all runs run at once and the makespan is that of
// the largest; at the small-molecule workload this beat equal-edge groups
// dispatched longest first.  Above kExactTargets targets a run holds many
// targets, so the granularity of whole targets (about three 32-edge chunks
// each at L = 5, 6) costs little without the exact refinement.
constexpr int kSchedThreads = 1024;
constexpr int kSchedItems = 8;

__device__ inline int runs_upto(int64_t X, int64_t W, int n_groups) {
  const int64_t r = ((X + 1) * n_groups + W - 1) / W;
  return r < n_groups ? (int)r : n_groups;
}

// One chunk of the fused kernel's greedy chunking (at most CM edges
// and kSlots targets per chunk) in a run that ends at target x (e_x =
// rp(x)): from edge e of target t (rp(t) <= e < rp(t + 1)) the chunk ends at
// min(e + CM, e_x, rp(min(t + kSlots, x))); t moves to the last target
// that starts at or before that end.  The kSlots row offsets are read at
// once; only targets without edges right at the end need the slow loop.
template <int CM, typename RP>
__device__ inline int chunk_end(const RP& rp, int& t, int e, int x, int e_x) {
  int r[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) r[j] = rp(min(t + 1 + j, x));
  const int e2 = min(min(e + CM, e_x), r[kSlots - 1]);
  int c = 0;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) c += r[j] <= e2;
  t += c;
  if (c == kSlots)
    while (t < x && rp(t + 1) <= e2) ++t;
  return e2;
}

// Chunks of run [s, x).
template <int CM, typename RP>
__device__ inline int run_chunks(const RP& rp, int s, int x) {
  int e = rp(s), t = s, c = 0;
  const int e_x = rp(x);
  if (e < e_x)
    while (rp(t + 1) <= e) ++t;
  while (e < e_x) {
    e = chunk_end<CM>(rp, t, e, x, e_x);
    ++c;
  }
  return c;
}

// Exact refinement for graphs of at most kExactTargets targets and
// kExactRuns runs.  The fused kernel's time per run is close to
// proportional to the run's chunk count, so the makespan is set by the
// largest count M of the estimated runs; with few chunks per run (about 18
// at the small-molecule workload) one chunk more on one run is a few
// percent.  Since greedy maximal
// chunks are the fewest for any range of targets, the chunk count of a
// range grows with the range, and the greedy partition under a cap of K
// chunks per run (each run as long as the cap allows) uses the fewest
// runs.  attn_groups_kernel counts the chunks of every estimated run (row
// offsets staged in LDS) and, when M exceeds the mean, sets K = M - 1;
// attn_runs_next_kernel finds, for every start s, the end next[s] of a
// greedy run of at most K chunks; attn_runs_chain_kernel follows the chain
// 0, next[0], next[next[0]], ... by pointer doubling and takes it as the
// run starts when n_groups runs reach n_targets, else keeps the estimate.
constexpr int kExactTargets = 12288;
constexpr int kExactRuns = 256;
constexpr int kExactItems = (kExactTargets + kSchedThreads) / kSchedThreads;  // row offsets per thread

// dst[i] = src[i] for i = 0..n1-1 (n1 <= kExactTargets + 1) by one workgroup
// of kSchedThreads, all loads in flight at once.
__device__ inline void stage_rows(const int32_t* __restrict__ src, int* dst, int n1) {
  int v[kExactItems];
#pragma unroll
  for (int k = 0; k < kExactItems; ++k) v[k] = src[min((int)threadIdx.x + k * kSchedThreads, n1 - 1)];
#pragma unroll
  for (int k = 0; k < kExactItems; ++k) {
    const int i = threadIdx.x + k * kSchedThreads;
    if (i < n1) dst[i] = v[k];
  }
}

template <bool EXACT, int CM>
__global__ void __launch_bounds__(kSchedThreads) attn_groups_kernel(const int32_t* __restrict__ row_ptr,
                                                                    int n_targets, int n_groups,
                                                                    int32_t* __restrict__ gs,
                                                                    int32_t* __restrict__ sched) {
  constexpr int kSpan = kSchedThreads * kSchedItems;
  __shared__ int64_t part[kSchedThreads / 64];
  __shared__ int wbuf[kSpan + kSpan / 32];
  __shared__ int gsl[kExactRuns + 1];  // run starts, exact refinement only
  __shared__ int red[2][kSchedThreads / 64];
  extern __shared__ int rps[];         // row_ptr, exact refinement only
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  if constexpr (EXACT) {
    stage_rows(row_ptr, rps, n_targets + 1);
    __syncthreads();
  }
  // row offsets from LDS in the exact mode, else from memory
  auto rp = [&](int i) {
    if constexpr (EXACT) return rps[i];
    else return row_ptr[i];
  };
  if constexpr (EXACT) {
    // all targets in one span: thread t takes targets kExactItems t ..
    // kExactItems t + kExactItems - 1, the block scan of the thread sums
    // gives both the prefixes and W
    const int i0 = t * kExactItems;
    int w[kExactItems];
    int64_t v = 0;
#pragma unroll
    for (int j = 0; j < kExactItems; ++j) {
      const int i = min(i0 + j, n_targets - 1);
      w[j] = i0 + j < n_targets ? (int)target_work<CM>(rp(i + 1) - rp(i)) : 0;
      v += w[j];
    }
    const int64_t own = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) part[wv] = v;
    __syncthreads();
    int64_t a = v - own, W = 0;
#pragma unroll
    for (int k = 0; k < kSchedThreads / 64; ++k) {
      if (k < wv) a += part[k];
      W += part[k];
    }
    if (t == 0) {
      gs[0] = gsl[0] = 0;
      gs[n_groups] = gsl[n_groups] = n_targets;
    }
    int g = runs_upto(a, W, n_groups);
#pragma unroll
    for (int j = 0; j < kExactItems; ++j) {
      a += w[j];
      if (i0 + j < n_targets)
        for (; g < n_groups && (int64_t)g * W < (a + 1) * n_groups; ++g) gs[g] = gsl[g] = i0 + j + 1;
    }
    __syncthreads();
  } else {
    // pass 1: W
    int64_t s = 0;
    for (int base = 0; base < n_targets; base += kSpan) {
      int d[kSchedItems];  // clamped, unpredicated loads: all in flight at once
#pragma unroll
      for (int j = 0; j < kSchedItems; ++j) {
        const int i = min(base + j * kSchedThreads + t, n_targets - 1);
        d[j] = rp(i + 1) - rp(i);
      }
#pragma unroll
      for (int j = 0; j < kSchedItems; ++j)
        if (base + j * kSchedThreads + t < n_targets) s += target_work<CM>(d[j]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) part[wv] = s;
    __syncthreads();
    int64_t W = 0;
#pragma unroll
    for (int k = 0; k < kSchedThreads / 64; ++k) W += part[k];
    __syncthreads();  // part is reused below

    if (t == 0) {
      gs[0] = 0;
      gs[n_groups] = n_targets;
    }

    // pass 2: targets i0 .. i0 + kSchedItems - 1 of each thread, their work
    // staged through LDS so that the row_ptr loads stay coalesced (the LDS
    // index is padded by one word per 32 to spread the reads over the banks)
    int64_t carry = 0;
    for (int base = 0; base < n_targets; base += kSpan) {
#pragma unroll
      for (int j = 0; j < kSchedItems; ++j) {
        const int i = min(base + j * kSchedThreads + t, n_targets - 1);
        const int dj = rp(i + 1) - rp(i);
        const int k = j * kSchedThreads + t;
        wbuf[k + (k >> 5)] = base + k < n_targets ? (int)target_work<CM>(dj) : 0;
      }
      __syncthreads();
      const int i0 = base + t * kSchedItems;
      int64_t w[kSchedItems];
      int64_t v = 0;
#pragma unroll
      for (int j = 0; j < kSchedItems; ++j) {
        const int k = t * kSchedItems + j;
        w[j] = wbuf[k + (k >> 5)];
        v += w[j];
      }
      // inclusive scan of the thread sums within the wave, then across waves
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
      }
      if (lane == 63) part[wv] = v;
      __syncthreads();
      int64_t a = carry, total = 0;
#pragma unroll
      for (int k = 0; k < kSchedThreads / 64; ++k) {
        if (k < wv) a += part[k];
        total += part[k];
      }
      a += __shfl_up(v, 1, 64) * (lane > 0);  // exclusive prefix of this thread
      // goal_g <= X  <=>  g W < (X + 1) n_groups: one division per thread
      int g = runs_upto(a, W, n_groups);
#pragma unroll
      for (int j = 0; j < kSchedItems; ++j) {
        const int i = i0 + j;
        a += w[j];
        if (i < n_targets)
          for (; g < n_groups && (int64_t)g * W < (a + 1) * n_groups; ++g) gs[g] = i + 1;
      }
      carry += total;
      __syncthreads();  // part is rewritten by the next span
    }
  }
  if constexpr (!EXACT) return;

  // chunk counts of the estimated runs: their maximum and sum set K
  int mx = t < n_groups ? run_chunks<CM>(rp, gsl[t], gsl[t + 1]) : 0;
  int sm = mx;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mx = max(mx, __shfl_xor(mx, off, 64));
    sm += __shfl_xor(sm, off, 64);
  }
  if (lane == 0) {
    red[0][wv] = mx;
    red[1][wv] = sm;
  }
  __syncthreads();
  if (t == 0) {
    int M = 0, S = 0;
    for (int k = 0; k < kSchedThreads / 64; ++k) {
      M = max(M, red[0][k]);
      S += red[1][k];
    }
    sched[0] = M > (S + n_groups - 1) / n_groups ? M - 1 : 0;
  }
}

// next[s] for s = 0..n_targets: the end of the greedy run from target s
// with at most K = sched[0] chunks (the first target that K chunks from
// row_ptr[s] do not finish), next[n_targets] = n_targets.  One thread per
// start; every workgroup stages all of row_ptr (at most kExactTargets + 1
// offsets) in LDS.
template <int CM>
__global__ void __launch_bounds__(kSchedThreads) attn_runs_next_kernel(const int32_t* __restrict__ row_ptr,
                                                                       int n_targets,
                                                                       const int32_t* __restrict__ sched,
                                                                       int32_t* __restrict__ next) {
  const int K = sched[0];
  if (K == 0) return;
  extern __shared__ int rpn[];  // n_targets + 1
  stage_rows(row_ptr, rpn, n_targets + 1);
  __syncthreads();
  auto rp = [&](int i) { return rpn[i]; };
  const int s = blockIdx.x * kSchedThreads + threadIdx.x;
  if (s > n_targets) return;
  const int e_end = rp(n_targets);
  int e = rp(s), t = s;
  if (e < e_end)
    while (rp(t + 1) <= e) ++t;
  for (int c = 0; c < K && e < e_end; ++c) e = chunk_end<CM>(rp, t, e, n_targets, e_end);
  next[s] = e < e_end ? t : n_targets;  // t holds edge e
}

// Run starts from next[]: next^2, next^4, next^8 and next^16 by squaring in
// LDS, the starts of runs 0, 16, 32, ... by one thread along next^16, the
// rest by one thread per 16 runs along next.  Written to gs only when run
// n_groups starts at n_targets (the cap K is feasible).
__global__ void __launch_bounds__(kSchedThreads) attn_runs_chain_kernel(const int32_t* __restrict__ next,
                                                                        int n_targets, int n_groups,
                                                                        const int32_t* __restrict__ sched,
                                                                        int32_t* __restrict__ gs) {
  if (sched[0] == 0) return;
  extern __shared__ int lds[];  // 3 (n_targets + 1)
  __shared__ int pos[kExactRuns + 1];
  const int t = threadIdx.x, n1 = n_targets + 1;
  int* A = lds;
  int* B = lds + n1;
  int* C = lds + 2 * n1;
  stage_rows(next, A, n1);
  __syncthreads();
  // Y = X o X, all gathers of a thread in flight at once
  auto square = [&](const int* X, int* Y) {
    int v[kExactItems];
#pragma unroll
    for (int k = 0; k < kExactItems; ++k) v[k] = X[min(t + k * kSchedThreads, n1 - 1)];
#pragma unroll
    for (int k = 0; k < kExactItems; ++k) v[k] = X[v[k]];
#pragma unroll
    for (int k = 0; k < kExactItems; ++k)
      if (t + k * kSchedThreads < n1) Y[t + k * kSchedThreads] = v[k];
    __syncthreads();
  };
  square(A, B);
  square(B, C);
  square(C, B);
  square(B, C);
  if (t == 0) {
    int x = 0;
    for (int j = 0; 16 * j <= n_groups; ++j) {
      pos[16 * j] = x;
      x = C[x];
    }
  }
  __syncthreads();
  if (16 * t < n_groups) {
    int x = pos[16 * t];
    for (int r = 1; r < 16 && 16 * t + r <= n_groups; ++r) {
      x = A[x];
      pos[16 * t + r] = x;
    }
  }
  __syncthreads();
  if (pos[n_groups] == n_targets)
    for (int g = t; g < n_groups; g += kSchedThreads) gs[g] = pos[g];
}

// MM: the per-m maps stop at |m| = MM (m_max; L for the base layer).
// F: focus streams (1: one; 2, 4, 8 at L <= 4 with the block-diagonal
// weights and the cross-focus softmax of focus_weights).
template <int L, int MM, int F>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
attn_mfma_kernel(MfmaParams P, int n_groups) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Smem<L>& S = *(Smem<L>*)smem;
  uint32_t* sD = (uint32_t*)(smem + Lds<L>::kD);
  float* sG = (float*)(smem + Lds<L>::kG);
  float* sW = (float*)(smem + Lds<L>::kW);
  float* sPhi = (float*)(smem + Lds<L>::kPhi);
  uint16_t* abase = (uint16_t*)(smem + Lds<L>::kA);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  constexpr int NC = Cfg<L>::NC;
  constexpr PassInfo p0 = pass_info(L, 0, MM);
  constexpr int NS0 = p0.M ? 2 : 1;
  constexpr int CM = Geo<L>::M, GL = Geo<L>::GL, MP = Geo<L>::MP;
  typedef typename XVec<Geo<L>::GCH>::type XV;

  // Workgroup -> group of consecutive targets (attn_groups_kernel and its
  // refinement chose the group starts).  Workgroups are dispatched to
  // the 8 XCDs round robin; XCD x takes a contiguous range of groups, since
  // neighbouring groups share neighbours in L2.
  const int b = blockIdx.x;
  const int grp = xcd_first(b % 8, n_groups) + b / 8;
  const int t_begin = P.gs[grp];
  const int t_end = P.gs[grp + 1];

  // targets without neighbours: y = 0, one wave per target
  for (int t = t_begin + wave; t < t_end; t += kWaves)
    if (P.row_ptr[t] == P.row_ptr[t + 1])
      for (int a = tid & 63; a < NC * kC; a += 64) P.y[(int64_t)t * NC * kC + a] = 0.0f;

  static_assert(16 * Cfg<L>::TT <= (int)(sizeof(S.rowinfo) / sizeof(S.rowinfo[0])), "row table");
  if (tid < 16 * Cfg<L>::TT) S.rowinfo[tid] = row_info(tid, Cfg<L>::TROWS);

  f32x4 T[Cfg<L>::TT][kNT];
#pragma unroll
  for (int ot = 0; ot < Cfg<L>::TT; ++ot)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) T[ot][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int e_end = P.row_ptr[t_end];
  int e = P.row_ptr[t_begin];
  int t_cur = t_begin;
  const int H = P.H;
  const int dh = kC / H;
  const float inv_sqrt_d = 1.0f / sqrtf((float)dh);
  const float rc = P.cutoff;
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(P.wf, P.w_bytes);
  const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(P.xp, P.xp_bytes);

  Ctx c;
  c.r0 = tid / GL;
  c.c8 = tid % GL;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) c.head[nt] = (16 * kNT * wave + 16 * nt + (tid & 15)) / dh;

  while (e < e_end) {
    while (P.row_ptr[t_cur + 1] <= e) ++t_cur;  // target of edge e
    const int t_first = t_cur;
    const int t_lim = min(t_first + kSlots, t_end);
    const int e_stop = min(min(e + CM, e_end), P.row_ptr[t_lim]);
    const int nrows = e_stop - e;

    // B fragments of the first pass's first K step go out before the setup
    u32x4 ring[2][p0.ND][n_bmat(p0.M)][kNT];
    {
      uint32_t boff[p0.ND][kNT];
      b_offsets<L, p0.M, p0.LO, p0.ND>(boff);
      load_b<L, p0.M, p0.LO, p0.ND>(wrs, boff, 0, ring[0]);
    }

    // ---- phase A1: per-edge metadata, radial basis and softmax weights
    if (tid <= kSlots) S.rp[tid] = P.row_ptr[min(t_first + tid, t_end)];
    __syncthreads();
    if (tid < kSlots) {
      int sl = 0;  // target of the chunk's last edge: t_first + sl
      while (sl + 1 < kSlots && S.rp[sl + 1] <= e_stop - 1) ++sl;
      const int t = t_first + ((tid - t_first % kSlots + kSlots) % kSlots);
      S.flush_t[tid] = (t <= t_first + sl && S.rp[t - t_first + 1] <= e_stop) ? t : -1;
    }
    {
      // GL lanes per edge row: lane 0 of row r computes the row's geometry
      // (in fp64) and stores the row metadata, then lane hs of the row
      // computes the radial basis functions hs, hs + GL, ... and the softmax
      // weights of heads hs, hs + GL, ... from the length and envelope it
      // reads from lane 0
      const int r = tid / GL, hs = tid % GL;
      int jr = -1;  // source atom of row r
      if (r < nrows) {
        int t, j;
        row_edge(S, e + r, t_first, t);
        j = P.col[e + r];
        jr = j;
        float rho = 0.0f, u = 0.0f;
        if (hs == 0) {
          const EdgeGeo geo = edge_geometry(P.pos, t, j, P.periodic, P.box, P.cutoff);
          rho = geo.rho;
          u = envelope_u(geo.s, geo.t, P.p);
          S.row_j[r] = j;
          S.row_slot[r] = t % kSlots;
          S.row_t[r] = t;
          S.row_rv[r] = f32x4{geo.r[0], geo.r[1], geo.r[2], rho};
          S.row_u[r] = u;
        }
        // every lane of the row is in this branch, so lane 0 of it is active
        const int src = (tid & 63) & ~(GL - 1);
        rho = __shfl(rho, src, 64);
        u = __shfl(u, src, 64);
        // Gaussian radial basis of this edge (centres k rc/(K-1), width rc/(K-1))
        const float step = rc / (float)(P.K - 1);
        const float inv2s2 = 1.0f / (2.0f * step * step);
        for (int kk = hs; kk < ((P.K + 7) & ~7); kk += GL) {
          const float dr = rho - step * (float)kk;
          sPhi[r * kMaxRbf + kk] = kk < P.K ? expf(-dr * dr * inv2s2) : 0.0f;
        }
        for (int h = hs; h < H; h += GL) {
          const f32x4* qv = (const f32x4*)(P.q + (int64_t)t * kC + h * dh);
          const f32x4* kv = (const f32x4*)(P.k + (int64_t)j * kC + h * dh);
          float z = 0.0f;
          for (int cc = 0; cc < dh / 4; ++cc) {
            const f32x4 qa = qv[cc], kb = kv[cc];
            z += qa.x * kb.x + qa.y * kb.y + qa.z * kb.z + qa.w * kb.w;
          }
          z = z * inv_sqrt_d + logit_bias(P, rho, h);
          sW[h * CM + r] = u * expf(z - P.stat_max[(int64_t)t * H + h]) * P.stat_inv[(int64_t)t * H + h];
        }
      } else {
        if (hs == 0) {
          S.row_j[r] = -1;
          S.row_slot[r] = -2;  // matches no slot
          S.row_t[r] = t_first;
          S.row_rv[r] = f32x4{0.0f, 0.0f, 1.0f, 0.0f};
          S.row_u[r] = 0.0f;
        }
        for (int kk = hs; kk < ((P.K + 7) & ~7); kk += GL) sPhi[r * kMaxRbf + kk] = 0.0f;
        for (int h = hs; h < H; h += GL) sW[h * CM + r] = 0.0f;
      }
      // the generator row of this lane is r (kGR = 1)
      static_assert(kGR == 1, "one generator row per lane, the phase A1 row");
      c.xoff[0] = jr >= 0 ? ((uint32_t)jr * Cfg<L>::NP * kC + Geo<L>::GCH * c.c8) * 4u : P.xp_bytes;
    }
    __syncthreads();

    // gathers of the first A chunk's generator units 0 and 1, which land
    // during phase A2
    XV xa[kGR * MP], xb[kGR * MP];
    gen_issue<L>(xrs, c, P.xp_bytes, p0.M, 0, xa);
    gen_issue<L>(xrs, c, P.xp_bytes, p0.M, 1, xb);

    // ---- phase A2: wave 0 the Wigner-D pairs of its edge row; waves 1..7
    // the radial gates: lane (channel quad cq, row phase rg) owns rows rg,
    // rg + NRG, ...; the w_rad columns of its 4 channels stream through
    // registers 8 basis functions at a time and meet every owned row
    float* s1 = (float*)(smem + Lds<L>::kS1);
    float* s4 = (float*)(smem + Lds<L>::kS4);
    float* s5 = (float*)(smem + Lds<L>::kS5);
    if (tid < 64) {
      const int r = tid;
      if (r < CM) {
        uint32_t* dr = sD + r * Cfg<L>::DPW;
        if (r < nrows) {
          const f32x4 v = S.row_rv[r];
          const float inv = v.w > 0.0f ? 1.0f / v.w : 0.0f;
          float R[9];
          edge_frame(v.x * inv, v.y * inv, v.z * inv, R);
          wigner_pairs<L>(R, dr, s1 + 9 * r, s4 + 81 * r);
        } else {
          for (int q = 0; q < Cfg<L>::DPW; ++q) dr[q] = 0u;
        }
      }
    } else {
      const int tw = tid - 64;  // 0 .. kThreads - 65
      constexpr int NRG = (kThreads - 64) / (kC / 4);
      constexpr int kGRows = (CM + NRG - 1) / NRG;
      const int cq = tw % (kC / 4), rg = tw / (kC / 4);
      if (rg < NRG) {
        f32x4 g[kGRows];
#pragma unroll
        for (int i = 0; i < kGRows; ++i) g[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (!(P.flags & SO2_FLAG_NO_RADIAL)) {
          for (int k0 = 0; k0 < P.K; k0 += 8) {
            f32x4 w4[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
              w4[kk] = k0 + kk < P.K ? *(const f32x4*)(P.wrad + (int64_t)(k0 + kk) * kC + 4 * cq)
                                     : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < kGRows; ++i) {
              const int r = rg + NRG * i;
              if (r < CM) {
                const f32x4 f0 = *(const f32x4*)(sPhi + r * kMaxRbf + k0);
                const f32x4 f1 = *(const f32x4*)(sPhi + r * kMaxRbf + k0 + 4);
                g[i] += f0.x * w4[0] + f0.y * w4[1] + f0.z * w4[2] + f0.w * w4[3] +
                        f1.x * w4[4] + f1.y * w4[5] + f1.z * w4[6] + f1.w * w4[7];
              }
            }
          }
        }
        const bool env = (P.flags & SO2_FLAG_RBF_ENVELOPE) != 0;
#pragma unroll
        for (int i = 0; i < kGRows; ++i) {
          const int r = rg + NRG * i;
          if (r < CM) {
            f32x4 gi = g[i];
            if (r >= nrows) gi = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            else if (P.flags & SO2_FLAG_NO_RADIAL) gi = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
            else if (env) gi = gi * S.row_u[r];
            *(f32x4*)(sG + g_off(r, cq)) = gi;
          }
        }
      }
    }
    __syncthreads();

    if constexpr (L >= 5) {
      // ---- phase A3 (L >= 5): D^5 and D^6 row by row, lane (row a, edge
      // er) of all waves, from the fp32 D^1, D^4 (and D^5) staged in the
      // idle A buffers; rows past the chunk's edges stay zero
      const int er = tid % CM, a = tid / CM;
      float D1[9];
      if (er < nrows) {
#pragma unroll
        for (int q = 0; q < 9; ++q) D1[q] = s1[9 * er + q];
        wigner_row_any<5, 0, (L >= 6)>(a, D1, s4 + 81 * er, sD + er * Cfg<L>::DPW, s5 + 121 * er);
      }
      __syncthreads();
      if constexpr (L >= 6) {
        if (er < nrows) wigner_row_any<6, 0, false>(a, D1, s5 + 121 * er, sD + er * Cfg<L>::DPW, nullptr);
        __syncthreads();
      }
    }

    // ---- focus streams: the cross-focus softmax folded into the weights
    if constexpr (F > 1) focus_weights<L, F>(P, smem, c, nrows);

    // ---- first A chunk (block p0.M, degree p0.M): all four generator units
    {
      uint32_t dp[kGR][MP], dm[kGR][MP];
      gen_dpairs<L>(sD, c, p0.M, p0.M, dp, dm);
      gen_finish<L, NS0>(sG, c, 0, xa, dp, dm, abase);  // chunks_before(L, 0, MM) = 0
      gen_issue<L>(xrs, c, P.xp_bytes, p0.M, 2, xa);
      gen_finish<L, NS0>(sG, c, 1, xb, dp, dm, abase);
      gen_issue<L>(xrs, c, P.xp_bytes, p0.M, 3, xb);
      gen_finish<L, NS0>(sG, c, 2, xa, dp, dm, abase);
      // gathers of generator unit 0 for chunk 0's target
      int gm, glp;
      gen_target<L, MM, 0>(0, gm, glp);
      gen_issue<L>(xrs, c, P.xp_bytes, glp, 0, xa);
      gen_finish<L, NS0>(sG, c, 3, xb, dp, dm, abase);

      // ---- phase B: every pass, each ending in its rotate-back GEMMs
      run_pass<L, MM, 0>(P, smem, c, T, ring, xa, xb);
    }

    // ---- phase D: write out targets whose last edge is in this chunk
    flush_slots<L>(P, S, t_first, T);
    e = e_stop;
  }
}

// One workgroup per compute unit, each with a run of consecutive targets
// holding an equal share of the estimated work (attn_groups_kernel, with the
// exact refinement on graphs of at most kExactTargets targets).
int group_count(int n_targets, int n_cu) { return std::max(1, std::min(n_cu, n_targets)); }

so2_status device_cu_count(int* n_cu) {
  int dev = 0;
  *n_cu = 256;
  SO2_CHECK(hipGetDevice(&dev));
  SO2_CHECK(hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  return SO2_OK;
}

// The run starts of the fused kernel.
template <int L>
so2_status schedule_L(const MfmaParams& P, int32_t* next, int32_t* sched, hipStream_t stream) {
  int n_cu = 256;
  const so2_status st = device_cu_count(&n_cu);
  if (st != SO2_OK) return st;
  const int n_groups = group_count(P.n_targets, n_cu);
  constexpr int CM = Geo<L>::M;
  const bool exact = P.n_targets <= kExactTargets && n_groups <= kExactRuns;
  if (exact) {
    const size_t lds1 = sizeof(int) * ((size_t)P.n_targets + 1);
    SO2_CHECK(hipFuncSetAttribute((const void*)(attn_groups_kernel<true, CM>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)(sizeof(int) * (kExactTargets + 1))));
    hipLaunchKernelGGL((attn_groups_kernel<true, CM>), dim3(1), dim3(kSchedThreads), lds1, stream, P.row_ptr,
                       P.n_targets, n_groups, const_cast<int32_t*>(P.gs), sched);
    SO2_CHECK_LAUNCH();
    hipLaunchKernelGGL(attn_runs_next_kernel<CM>, dim3((P.n_targets + kSchedThreads) / kSchedThreads),
                       dim3(kSchedThreads), lds1, stream, P.row_ptr, P.n_targets, (const int32_t*)sched, next);
    SO2_CHECK_LAUNCH();
    SO2_CHECK(hipFuncSetAttribute((const void*)attn_runs_chain_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)(3 * sizeof(int) * (kExactTargets + 1))));
    hipLaunchKernelGGL(attn_runs_chain_kernel, dim3(1), dim3(kSchedThreads), 3 * lds1, stream, (const int32_t*)next,
                       P.n_targets, n_groups, (const int32_t*)sched, const_cast<int32_t*>(P.gs));
  } else {
    hipLaunchKernelGGL((attn_groups_kernel<false, CM>), dim3(1), dim3(kSchedThreads), 0, stream, P.row_ptr,
                       P.n_targets, n_groups, const_cast<int32_t*>(P.gs), sched);
  }
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

template <int L, int MM, int F>
so2_status launch_instance(const MfmaParams& P, int n_groups, hipStream_t stream) {
  const size_t smem = Lds<L>::kTotal;
  static_assert(Lds<L>::kTotal <= 160 * 1024, "LDS budget");
  SO2_CHECK(hipFuncSetAttribute((const void*)attn_mfma_kernel<L, MM, F>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem));
  hipLaunchKernelGGL((attn_mfma_kernel<L, MM, F>), dim3(n_groups), dim3(kThreads), smem, stream, P, n_groups);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

// The kernel instance of P.m_max (MM counts down from L), one stream.
template <int L, int MM>
so2_status launch_LM(const MfmaParams& P, int n_groups, hipStream_t stream) {
  if constexpr (MM > 0) {
    if (P.m_max < MM) return launch_LM<L, MM - 1>(P, n_groups, stream);
  }
  if (P.m_max != MM) return SO2_ERR_INVALID_ARGUMENT;
  return launch_instance<L, MM, 1>(P, n_groups, stream);
}

template <int L>
so2_status launch_L(const MfmaParams& P, hipStream_t stream) {
  int n_cu = 256;
  const so2_status st = device_cu_count(&n_cu);
  if (st != SO2_OK) return st;
  const int n_groups = group_count(P.n_targets, n_cu);
  if (P.n_focus == 1) return launch_LM<L, L>(P, n_groups, stream);
  if constexpr (L <= 4) {
    if (P.m_max != L || P.H % P.n_focus) return SO2_ERR_INVALID_ARGUMENT;
    switch (P.n_focus) {
      case 2:
        return launch_instance<L, L, 2>(P, n_groups, stream);
      case 4:
        return launch_instance<L, L, 4>(P, n_groups, stream);
      case 8:
        return launch_instance<L, L, 8>(P, n_groups, stream);
    }
  }
  return SO2_ERR_INVALID_ARGUMENT;
}

// Workspace of the MFMA path: softmax statistics, the x pairs, w_rad in
// fp32 and w_so2 in fragment order.
struct ScratchLayout {
  size_t stats, xp, wrad, wf, gs, next, sched, total;
};

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

ScratchLayout scratch_layout(int n_atoms, int n_targets, int L, int H, int K) {
  ScratchLayout s{};
  s.stats = 0;
  s.xp = up256(sizeof(float) * 2 * (size_t)n_targets * H);
  s.wrad = s.xp + up256(sizeof(uint32_t) * (size_t)n_atoms * pair_off(L + 1) * kC);
  s.wf = s.wrad + up256(sizeof(float) * (size_t)K * kC);
  s.gs = s.wf + up256(sizeof(uint16_t) * (size_t)wf_entries(L));
  // at most n_targets groups
  s.next = s.gs + up256(sizeof(int32_t) * ((size_t)n_targets + 1));
  s.sched = s.next + up256(sizeof(int32_t) * ((size_t)n_targets + 1));
  s.total = s.sched + 256;
  return s;
}

MfmaParams make_params(const AttnArgs& a) {
  MfmaParams P{};
  const ScratchLayout s = scratch_layout(a.n_atoms, a.n_targets, a.L, a.H, a.K);
  char* base = (char*)a.scratch;
  P.pos = a.pos;
  P.row_ptr = a.row_ptr;
  P.col = a.col;
  P.xp = (const uint32_t*)(base + s.xp);
  P.wrad = (const float*)(base + s.wrad);
  P.wf = (const uint16_t*)(base + s.wf);
  P.gs = (const int32_t*)(base + s.gs);
  P.q = a.q;
  P.k = a.k;
  float* stats = (float*)(base + s.stats);
  P.stat_max = stats;
  P.stat_inv = stats + (size_t)a.n_targets * a.H;
  P.y = a.y;
  P.w_logit = (const uint16_t*)a.w_logit;
  P.xp_bytes = (uint32_t)((uint64_t)a.n_atoms * pair_off(a.L + 1) * kC * 4);
  P.w_bytes = (uint32_t)(w1_offset(a.L, a.m_max + 1) * 2);  // the blocks m <= m_max (dense over the streams)
  P.m_max = a.m_max;
  P.n_focus = a.n_focus;
  P.w_focus = (const uint16_t*)a.w_focus;
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

template <int L>
so2_status launch_pack_L(const AttnArgs& a, const MfmaParams& P, hipStream_t stream) {
  // w_so2 holds the blocks m <= m_max, for each of the F streams over C / F channels
  const int F = a.n_focus;
  const int Cs = kC / F;
  int64_t w_entries = (int64_t)(L + 1) * Cs * (L + 1) * Cs;
  for (int m = 1; m <= a.m_max; ++m) w_entries += 2 * (int64_t)(L + 1 - m) * Cs * (L + 1 - m) * Cs;
  w_entries *= F;
  const int64_t work = (int64_t)a.n_atoms * pair_off(L + 1) * (kC / 4) + (int64_t)a.K * kC +
                       (F == 1 ? w_entries : wf_entries(L)) / 8;
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, 8192);
  hipLaunchKernelGGL(attn_pack_kernel<L>, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t*)a.x, const_cast<uint32_t*>(P.xp), a.n_atoms, (const uint16_t*)a.w_rad,
                     const_cast<float*>(P.wrad), a.K, (const uint16_t*)a.w_so2, const_cast<uint16_t*>(P.wf),
                     w_entries, F);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

}  // namespace

bool mfma_shape(int L, int C, int H, int K) {
  return C == kC && L >= 1 && L <= 6 && H >= 1 && H <= kMaxHeads && C % H == 0 && K <= kMaxRbf;
}

// Focus streams on the MFMA kernel: 64-edge chunks (L <= 4), every order,
// F of 2, 4 or 8 streams (whole waves of 16 channels each) dividing H.
bool mfma_focus(int L, int H, int m_max, int n_focus) {
  return n_focus == 1 || (L <= 4 && m_max == L && (n_focus == 2 || n_focus == 4 || n_focus == 8) && H % n_focus == 0);
}

// The x pairs are addressed through a 32-bit buffer descriptor, with room
// past the end for the zero reads of rows without an edge: 4 (L+1)(L+2)/2 C
// bytes per atom below 2^32 - 2^16 (about 559k atoms at L = 4, 299k at L = 6).
bool mfma_fits(int L, int n_atoms) {
  const uint64_t xp_bytes = (uint64_t)n_atoms * pair_off(L + 1) * kC * 4;
  return xp_bytes < 0xffff0000ull;
}

bool mfma_aligned(const AttnArgs& a) {
  return !(((uintptr_t)a.x & 15) || ((uintptr_t)a.w_so2 & 15) || ((uintptr_t)a.w_rad & 15));
}

size_t mfma_scratch_bytes(int n_atoms, int n_targets, int L, int H, int K) {
  return scratch_layout(n_atoms, n_targets, L, H, K).total;
}

namespace {

so2_status launch_schedule(const AttnArgs& a, const MfmaParams& P, hipStream_t stream) {
  const ScratchLayout s = scratch_layout(a.n_atoms, a.n_targets, a.L, a.H, a.K);
  int32_t* next = (int32_t*)((char*)a.scratch + s.next);
  int32_t* sched = (int32_t*)((char*)a.scratch + s.sched);
  switch (a.L) {
    case 1:
      return schedule_L<1>(P, next, sched, stream);
    case 2:
      return schedule_L<2>(P, next, sched, stream);
    case 3:
      return schedule_L<3>(P, next, sched, stream);
    case 4:
      return schedule_L<4>(P, next, sched, stream);
    case 5:
      return schedule_L<5>(P, next, sched, stream);
    case 6:
      return schedule_L<6>(P, next, sched, stream);
  }
  return SO2_ERR_UNSUPPORTED;
}

}  // namespace

// Prologue of the fused kernel, in order on the caller's stream: the run
// schedule (reads only row_ptr), the repack of x and the weights, and the
// softmax statistics.
so2_status launch_attention_mfma_prep(const AttnArgs& a, hipStream_t stream) {
  const MfmaParams P = make_params(a);
  if (a.n_targets > 0) {
    const so2_status st = launch_schedule(a, P, stream);
    if (st != SO2_OK) return st;
  }
  so2_status st = SO2_OK;
  switch (a.L) {
    case 1:
      st = launch_pack_L<1>(a, P, stream);
      break;
    case 2:
      st = launch_pack_L<2>(a, P, stream);
      break;
    case 3:
      st = launch_pack_L<3>(a, P, stream);
      break;
    case 4:
      st = launch_pack_L<4>(a, P, stream);
      break;
    case 5:
      st = launch_pack_L<5>(a, P, stream);
      break;
    case 6:
      st = launch_pack_L<6>(a, P, stream);
      break;
    default:
      st = SO2_ERR_UNSUPPORTED;
  }
  if (st == SO2_OK && a.n_targets > 0) {
    hipLaunchKernelGGL(attn_stats_kernel, dim3((a.n_targets + 3) / 4), dim3(256), 0, stream, P, kC);
    SO2_CHECK_LAUNCH();
  }
  return st;
}

so2_status launch_attention_mfma(const AttnArgs& a, hipStream_t stream) {
  if (a.n_targets == 0) return SO2_OK;
  const MfmaParams P = make_params(a);
  switch (a.L) {
    case 1:
      return launch_L<1>(P, stream);
    case 2:
      return launch_L<2>(P, stream);
    case 3:
      return launch_L<3>(P, stream);
    case 4:
      return launch_L<4>(P, stream);
    case 5:
      return launch_L<5>(P, stream);
    case 6:
      return launch_L<6>(P, stream);
  }
  return SO2_ERR_UNSUPPORTED;
}

}  // namespace so2
