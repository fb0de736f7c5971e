// Cell-list radius graph for gfx950.
//
// The E2Former-V2 summary (technical section 2.2) streams, for every atom
// i, its neighbours j in N(i) within a cutoff radius; the pages assume N(i)
// is given.  This builder produces it as CSR, bit-identical to a brute-force
// search that uses the same fp64 operation sequence (see so2attn.h).
//
// Pipeline (all on the caller's stream):
//   bbox      one workgroup: min/max of the positions, count of non-finite
//             values -> host (sync 1) -> host picks the cell grid
//   assign    cell of every atom, cell occupancy (atomics)
//   scan      occupancy -> cell start (one workgroup)
//   scatter   atoms grouped by cell, with their positions and molecule ids
//   count     16 lanes per atom: up to 27 cells, exact fp64 test
//   scan      counts -> row_ptr, E as int64 -> host (sync 2)
//   fill      same loop, writes col (order within a row is arbitrary)
//   sort      ascending j inside each row: one 64-lane workgroup per row up
//             to 1024 entries (bitonic in LDS), one 1024-lane workgroup per
//             longer row up to 16384 entries
//
// The fp64 distance arithmetic must not be contracted into FMAs: the test
// must round every operation exactly like the brute-force definition.
#pragma clang fp contract(off)

#include <math.h>

#include "common.h"
#include "launch.h"

namespace so2 {

constexpr int kShortRow = 1024;
constexpr int kLongRow = 16384;

struct GridParams {
  double origin[3];
  double inv_cell[3];
  double box[3];
  int n[3];
  int periodic;
};

// Cells at least rc wide (widened by 1e-6 so that rounding of the cell
// coordinate can never split a pair closer than rc by two cells), at most
// max_cells of them: the longest axis is halved until the grid fits.
__device__ inline void make_grid(const float* bb, double rc, int periodic, const double* box, int64_t max_cells,
                                 GridParams& g) {
  const double cs = rc * (1.0 + 1e-6);
  g.periodic = periodic;
  for (int d = 0; d < 3; ++d) {
    if (periodic) {
      g.box[d] = box[d];
      g.origin[d] = 0.0;
      g.n[d] = (int)fmax(1.0, floor(box[d] / cs));
    } else {
      const double ext = (double)bb[3 + d] - (double)bb[d];
      g.box[d] = 0.0;
      g.origin[d] = (double)bb[d];
      g.n[d] = (int)fmax(1.0, fmin(floor(ext / cs), 1e9));
    }
  }
  while ((int64_t)g.n[0] * g.n[1] * g.n[2] > max_cells) {
    const int d = (g.n[0] >= g.n[1] && g.n[0] >= g.n[2]) ? 0 : (g.n[1] >= g.n[2] ? 1 : 2);
    g.n[d] = (g.n[d] + 1) / 2;
  }
  for (int d = 0; d < 3; ++d) {
    const double cell = periodic ? g.box[d] / g.n[d] : fmax(cs, ((double)bb[3 + d] - (double)bb[d]) / g.n[d]);
    g.inv_cell[d] = 1.0 / cell;
  }
}

// Bounding box of the finite coordinates, a flag for non-finite ones, and
// the cell grid built from them (or from the box), all written to device
// memory: no host round trip before the binning.  Non-finite coordinates
// still land in clamped cells (NaN converts to 0, +-inf saturates), so every
// later kernel stays in bounds; the call reports them once E is read back.
__global__ void __launch_bounds__(1024) nb_bbox_kernel(const float* __restrict__ pos, int n,
                                                      float* __restrict__ out_f,
                                                      int* __restrict__ out_i, double rc, int periodic,
                                                      double bx, double by, double bz, long long max_cells,
                                                      GridParams* __restrict__ out_g,
                                                      int* __restrict__ out_ncell) {
  __shared__ float s_mn[3][1024];
  __shared__ float s_mx[3][1024];
  __shared__ int s_bad[1024];
  int t = threadIdx.x;
  float mn[3] = {INFINITY, INFINITY, INFINITY};
  float mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  int bad = 0;
  for (int i = t; i < n; i += blockDim.x) {
    for (int d = 0; d < 3; ++d) {
      float v = pos[3 * (int64_t)i + d];
      if (!isfinite(v)) {
        bad = 1;
        continue;
      }
      mn[d] = fminf(mn[d], v);
      mx[d] = fmaxf(mx[d], v);
    }
  }
  for (int d = 0; d < 3; ++d) {
    s_mn[d][t] = mn[d];
    s_mx[d][t] = mx[d];
  }
  s_bad[t] = bad;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if (t < s) {
      for (int d = 0; d < 3; ++d) {
        s_mn[d][t] = fminf(s_mn[d][t], s_mn[d][t + s]);
        s_mx[d][t] = fmaxf(s_mx[d][t], s_mx[d][t + s]);
      }
      s_bad[t] |= s_bad[t + s];
    }
    __syncthreads();
  }
  if (t == 0) {
    float bb[6];
    for (int d = 0; d < 3; ++d) {
      bb[d] = s_mn[d][0];
      bb[3 + d] = s_mx[d][0];
    }
    const double box[3] = {bx, by, bz};
    GridParams g;
    make_grid(bb, rc, periodic, box, max_cells, g);
    *out_g = g;
    *out_ncell = g.n[0] * g.n[1] * g.n[2];
    for (int d = 0; d < 3; ++d) {
      out_f[d] = s_mn[d][0];
      out_f[3 + d] = s_mx[d][0];
    }
    out_i[0] = s_bad[0];
  }
}

__device__ inline int cell_coord(double p, int d, const GridParams& g) {
  double w;
  if (g.periodic) {
    w = p - g.box[d] * floor(p / g.box[d]);
  } else {
    w = p - g.origin[d];
  }
  int c = (int)floor(w * g.inv_cell[d]);
  c = c < 0 ? 0 : c;
  c = c >= g.n[d] ? g.n[d] - 1 : c;
  return c;
}

__global__ void nb_assign_kernel(const float* __restrict__ pos, int n, const GridParams* __restrict__ gp,
                                 int* __restrict__ cell_of, int* __restrict__ cell_count) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const GridParams g = *gp;
  int cx = cell_coord((double)pos[3 * (int64_t)i + 0], 0, g);
  int cy = cell_coord((double)pos[3 * (int64_t)i + 1], 1, g);
  int cz = cell_coord((double)pos[3 * (int64_t)i + 2], 2, g);
  int c = (cz * g.n[1] + cy) * g.n[0] + cx;
  cell_of[i] = c;
  atomicAdd(&cell_count[c], 1);
}

// Exclusive scan of in[0..n) into out[0..n] (and out2[0..n) if given),
// out[n] = total (int32), total also stored as int64 in *total64; n is read
// from n_dev when that is given.  One workgroup of 1024 threads walks the
// input in spans of 8192 values.  A span is loaded with coalesced loads into
// LDS; each thread then takes 8 consecutive values, the thread sums are
// scanned with wave shuffles and across the 16 waves, the results go back
// through LDS and out with coalesced stores; a running carry links the
// spans.  The LDS index is padded by one word per 32 so that the
// consecutive-value reads of a wave spread over the banks.
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 8;
constexpr int kScanSpan = kScanThreads * kScanItems;
__device__ inline int scan_pad(int i) { return i + (i >> 5); }

__global__ void __launch_bounds__(kScanThreads) nb_scan_kernel(const int* __restrict__ in, int n,
                                                               const int* __restrict__ n_dev, int* __restrict__ out,
                                                               int* __restrict__ out2, long long* __restrict__ total64) {
  __shared__ long long part[kScanThreads / 64];
  __shared__ int buf[kScanSpan + kScanSpan / 32];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  if (n_dev) n = *n_dev;
  long long carry = 0;
  for (int base = 0; base < n; base += kScanSpan) {
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      const int i = base + j * kScanThreads + t;
      const int x = in[min(i, n - 1)];
      buf[scan_pad(j * kScanThreads + t)] = i < n ? x : 0;
    }
    __syncthreads();
    int v[kScanItems];
    long long sum = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      v[j] = buf[scan_pad(t * kScanItems + j)];
      sum += v[j];
    }
    long long incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) part[wv] = incl;
    __syncthreads();
    long long run = carry + incl - sum, total = 0;
#pragma unroll
    for (int k = 0; k < kScanThreads / 64; ++k) {
      if (k < wv) run += part[k];
      total += part[k];
    }
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      buf[scan_pad(t * kScanItems + j)] = (int)run;
      run += v[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      const int i = base + j * kScanThreads + t;
      if (i < n) {
        const int r = buf[scan_pad(j * kScanThreads + t)];
        out[i] = r;
        if (out2) out2[i] = r;
      }
    }
    carry += total;
    __syncthreads();  // part and buf are rewritten by the next span
  }
  if (t == 0) {
    out[n] = (int)carry;
    if (total64) *total64 = carry;
  }
}

__global__ void nb_scatter_kernel(const float* __restrict__ pos, const int* __restrict__ mol,
                                  int n, const int* __restrict__ cell_of,
                                  int* __restrict__ cursor, int* __restrict__ sorted_idx,
                                  float* __restrict__ sorted_pos, int* __restrict__ sorted_mol) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int k = atomicAdd(&cursor[cell_of[i]], 1);
  sorted_idx[k] = i;
  sorted_pos[3 * (int64_t)k + 0] = pos[3 * (int64_t)i + 0];
  sorted_pos[3 * (int64_t)k + 1] = pos[3 * (int64_t)i + 1];
  sorted_pos[3 * (int64_t)k + 2] = pos[3 * (int64_t)i + 2];
  sorted_mol[k] = mol ? mol[i] : 0;
}

// Unique neighbour cell offsets along one axis (handles grids of 1 or 2
// cells in a periodic direction, where -1 and +1 name the same cell).
__device__ inline int axis_cells(int c, int d, const GridParams& g, int* out) {
  int cnt = 0;
  for (int o = -1; o <= 1; ++o) {
    int v = c + o;
    if (g.periodic) {
      v = (v % g.n[d] + g.n[d]) % g.n[d];
    } else if (v < 0 || v >= g.n[d]) {
      continue;
    }
    bool dup = false;
    for (int q = 0; q < cnt; ++q) dup |= (out[q] == v);
    if (!dup) out[cnt++] = v;
  }
  return cnt;
}

// The exact neighbour test (see so2attn.h); fp contraction is off in this file.
__device__ inline bool within_cutoff(double pix, double piy, double piz, double pjx, double pjy,
                                     double pjz, const GridParams& g, double rc2) {
  double dx = pjx - pix;
  double dy = pjy - piy;
  double dz = pjz - piz;
  if (g.periodic) {
    dx = dx - g.box[0] * rint(dx / g.box[0]);
    dy = dy - g.box[1] * rint(dy / g.box[1]);
    dz = dz - g.box[2] * rint(dz / g.box[2]);
  }
  double s = (dx * dx + dy * dy) + dz * dz;
  return s < rc2;
}

// Count (kFill = false) or fill (kFill = true) the neighbours of atom i with
// kGroup lanes per atom: the group walks the up to 27 cells together, its
// lanes taking the cell's members kGroup apart, and counts its hits with a
// ballot; in the fill pass every hit goes to row_ptr[i] + (hits so far) +
// (hits of lower lanes of the group in this round).
constexpr int kGroup = 16;
template <bool kFill>
__global__ void __launch_bounds__(256) nb_pairs_kernel(const float* __restrict__ pos, const int* __restrict__ mol,
                                                       int n, const GridParams* __restrict__ gp, double rc2,
                                                       const int* __restrict__ cell_start,
                                                       const int* __restrict__ sorted_idx,
                                                       const float* __restrict__ sorted_pos,
                                                       const int* __restrict__ sorted_mol, int* __restrict__ counts,
                                                       const int* __restrict__ row_ptr, int* __restrict__ col,
                                                       int* __restrict__ long_rows, int* __restrict__ n_long,
                                                       int* __restrict__ n_over) {
  const int gid = blockIdx.x * (blockDim.x / kGroup) + threadIdx.x / kGroup;
  const int li = threadIdx.x % kGroup;                // lane within the group
  const int gshift = (threadIdx.x & 63) & ~(kGroup - 1);  // first lane of the group in the wave
  if (gid >= n) return;  // whole groups leave together
  const GridParams g = *gp;
  const int i = gid;
  const double pix = (double)pos[3 * (int64_t)i + 0];
  const double piy = (double)pos[3 * (int64_t)i + 1];
  const double piz = (double)pos[3 * (int64_t)i + 2];
  const int mi = mol ? mol[i] : 0;
  int cx[3], cy[3], cz[3];
  const int nx = axis_cells(cell_coord(pix, 0, g), 0, g, cx);
  const int ny = axis_cells(cell_coord(piy, 1, g), 1, g, cy);
  const int nz = axis_cells(cell_coord(piz, 2, g), 2, g, cz);
  int cnt = 0;  // hits of the whole group so far (same in every lane)
  const int base = kFill ? row_ptr[i] : 0;
  for (int a = 0; a < nz; ++a)
    for (int b = 0; b < ny; ++b)
      for (int c = 0; c < nx; ++c) {
        const int cell = (cz[a] * g.n[1] + cy[b]) * g.n[0] + cx[c];
        const int k0 = cell_start[cell], k1 = cell_start[cell + 1];
        for (int kb = k0; kb < k1; kb += kGroup) {
          const int k = kb + li;
          bool hit = false;
          int j = -1;
          if (k < k1) {
            j = sorted_idx[k];
            if (j != i && sorted_mol[k] == mi) {
              const double pjx = (double)sorted_pos[3 * (int64_t)k + 0];
              const double pjy = (double)sorted_pos[3 * (int64_t)k + 1];
              const double pjz = (double)sorted_pos[3 * (int64_t)k + 2];
              hit = within_cutoff(pix, piy, piz, pjx, pjy, pjz, g, rc2);
            }
          }
          const unsigned long long bal = __ballot(hit);
          const unsigned int gm = (unsigned int)(bal >> gshift) & ((1u << kGroup) - 1u);
          if (kFill && hit) col[base + cnt + __popc(gm & ((1u << li) - 1u))] = j;
          cnt += __popc(gm);
        }
      }
  if (!kFill && li == 0) {
    counts[i] = cnt;
    if (cnt > kLongRow) {
      atomicAdd(n_over, 1);
    } else if (cnt > kShortRow) {
      int slot = atomicAdd(n_long, 1);
      long_rows[slot] = i;
    }
  }
}

// Bitonic sort (every comparator ascending; the first step of each stage
// compares i with i ^ (k-1)), keys padded with INT_MAX to a power of two.
__device__ inline void bitonic_lds(int* s, int P, int t, int nthreads) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int q = t; q < P / 2; q += nthreads) {
        // q-th pair of this step: lower index i has bit j clear
        int i = ((q / j) * 2 * j) + (q % j);
        int partner = (j == (k >> 1)) ? (i ^ (k - 1)) : (i + j);
        int lo = min(i, partner), hi = max(i, partner);
        int a = s[lo], b = s[hi];
        if (a > b) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(64) nb_sort_short_kernel(const int* __restrict__ row_ptr,
                                                          int* __restrict__ col, int n) {
  __shared__ int s[kShortRow];
  int i = blockIdx.x;
  if (i >= n) return;
  int a = row_ptr[i], len = row_ptr[i + 1] - a;
  if (len <= 1 || len > kShortRow) return;
  int P = 2;
  while (P < len) P <<= 1;
  for (int k = threadIdx.x; k < P; k += 64) s[k] = (k < len) ? col[a + k] : 0x7fffffff;
  __syncthreads();
  bitonic_lds(s, P, threadIdx.x, 64);
  for (int k = threadIdx.x; k < len; k += 64) col[a + k] = s[k];
}

__global__ void __launch_bounds__(1024) nb_sort_long_kernel(const int* __restrict__ row_ptr,
                                                           int* __restrict__ col,
                                                           const int* __restrict__ long_rows) {
  __shared__ int s[kLongRow];
  int i = long_rows[blockIdx.x];
  int a = row_ptr[i], len = row_ptr[i + 1] - a;
  int P = 2;
  while (P < len) P <<= 1;
  for (int k = threadIdx.x; k < P; k += 1024) s[k] = (k < len) ? col[a + k] : 0x7fffffff;
  __syncthreads();
  bitonic_lds(s, P, threadIdx.x, 1024);
  for (int k = threadIdx.x; k < len; k += 1024) col[a + k] = s[k];
}

// ------------------------------------------------------------------ host

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int64_t max_cells(int32_t n_atoms) { return 2 * (int64_t)n_atoms + 1024; }

struct NbLayout {
  size_t bbox, grid, cell_of, cell_count, cell_start, cursor, sorted_idx, sorted_pos, sorted_mol,
      counts, long_rows, scalars, total;
};

NbLayout nb_layout(int32_t n) {
  NbLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  int64_t nc = max_cells(n);
  L.bbox = take(64);
  L.grid = take(sizeof(GridParams) + 16);
  L.cell_of = take(sizeof(int) * (size_t)n);
  L.cell_count = take(sizeof(int) * (size_t)(nc + 1));
  L.cell_start = take(sizeof(int) * (size_t)(nc + 1));
  L.cursor = take(sizeof(int) * (size_t)(nc + 1));
  L.sorted_idx = take(sizeof(int) * (size_t)n);
  L.sorted_pos = take(sizeof(float) * 3 * (size_t)n);
  L.sorted_mol = take(sizeof(int) * (size_t)n);
  L.counts = take(sizeof(int) * (size_t)n);
  L.long_rows = take(sizeof(int) * (size_t)n);
  L.scalars = take(64);  // [0] E (int64), [8] n_long, [12] n_over, [16] non-finite flag
  L.total = off;
  return L;
}

__global__ void nb_zero_kernel(int* __restrict__ p, int64_t n) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

size_t neighbors_workspace_bytes(int32_t n_atoms) {
  if (n_atoms < 1) return 0;
  return nb_layout(n_atoms).total;
}

so2_status neighbors_build(const float* pos, int32_t n, const int32_t* mol_id,
                           const float* box_host, float cutoff, int32_t* row_ptr, int32_t* col,
                           int64_t capacity, int64_t* n_edges_host, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  const NbLayout L = nb_layout(n);
  if (workspace_bytes < L.total || ((uintptr_t)workspace & 255)) return SO2_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  float* bbox_f = (float*)(ws + L.bbox);
  int* cell_of = (int*)(ws + L.cell_of);
  int* cell_count = (int*)(ws + L.cell_count);
  int* cell_start = (int*)(ws + L.cell_start);
  int* cursor = (int*)(ws + L.cursor);
  int* sorted_idx = (int*)(ws + L.sorted_idx);
  float* sorted_pos = (float*)(ws + L.sorted_pos);
  int* sorted_mol = (int*)(ws + L.sorted_mol);
  int* counts = (int*)(ws + L.counts);
  int* long_rows = (int*)(ws + L.long_rows);
  long long* e_total = (long long*)(ws + L.scalars);
  int* n_long = (int*)(ws + L.scalars + 8);
  int* n_over = (int*)(ws + L.scalars + 12);

  GridParams* grid = (GridParams*)(ws + L.grid);
  int* ncell_dev = (int*)(ws + L.grid + sizeof(GridParams));
  int* bad_dev = (int*)(ws + L.scalars + 16);
  const int64_t ncell_max = max_cells(n);

  // 1. bounding box, finiteness flag and cell grid, on the device
  hipLaunchKernelGGL(nb_zero_kernel, dim3(1), dim3(64), 0, stream, (int*)(ws + L.scalars), 16);
  const int periodic = box_host != nullptr;
  hipLaunchKernelGGL(nb_bbox_kernel, dim3(1), dim3(1024), 0, stream, pos, n, bbox_f, bad_dev, (double)cutoff,
                     periodic, periodic ? (double)box_host[0] : 0.0, periodic ? (double)box_host[1] : 0.0,
                     periodic ? (double)box_host[2] : 0.0, (long long)ncell_max, grid, ncell_dev);
  SO2_CHECK_LAUNCH();
  const double rc = (double)cutoff;

  // 2.-3. bin atoms by cell (launch sizes from the cell bound; the kernels
  // read the grid and its cell count from device memory)
  const int tb = 256;
  const int nblk = (n + tb - 1) / tb;
  hipLaunchKernelGGL(nb_zero_kernel, dim3((unsigned)((ncell_max + 1 + 255) / 256)), dim3(256), 0, stream,
                     cell_count, (int64_t)ncell_max + 1);
  hipLaunchKernelGGL(nb_assign_kernel, dim3(nblk), dim3(tb), 0, stream, pos, n, (const GridParams*)grid, cell_of,
                     cell_count);
  hipLaunchKernelGGL(nb_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, cell_count, 0, (const int*)ncell_dev,
                     cell_start, cursor, (long long*)nullptr);
  hipLaunchKernelGGL(nb_scatter_kernel, dim3(nblk), dim3(tb), 0, stream, pos, mol_id, n, cell_of,
                     cursor, sorted_idx, sorted_pos, sorted_mol);
  SO2_CHECK_LAUNCH();

  // 4. count, scan, read E
  const double rc2 = rc * rc;
  const int nblk_pairs = (n + tb / kGroup - 1) / (tb / kGroup);
  hipLaunchKernelGGL(nb_pairs_kernel<false>, dim3(nblk_pairs), dim3(tb), 0, stream, pos, mol_id, n,
                     (const GridParams*)grid, rc2, cell_start, sorted_idx, sorted_pos, sorted_mol, counts,
                     (const int*)nullptr, (int*)nullptr, long_rows, n_long, n_over);
  hipLaunchKernelGGL(nb_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts, n, (const int*)nullptr, row_ptr,
                     (int*)nullptr, e_total);
  SO2_CHECK_LAUNCH();
  long long hs[3] = {0, 0, 0};
  SO2_CHECK(hipMemcpyAsync(hs, e_total, 24, hipMemcpyDeviceToHost, stream));
  SO2_CHECK(hipStreamSynchronize(stream));
  if (hs[2] & 0xffffffffLL) return SO2_ERR_INVALID_ARGUMENT;  // non-finite positions
  const long long E = hs[0];
  const int h_long = (int)(hs[1] & 0xffffffffLL);
  const int h_over = (int)((unsigned long long)hs[1] >> 32);
  *n_edges_host = E;
  if (E > 0x7fffffffLL) return SO2_ERR_INVALID_ARGUMENT;
  if (h_over > 0) return SO2_ERR_UNSUPPORTED;
  if (E > capacity) return SO2_ERR_CAPACITY;

  // 5. fill and sort rows
  hipLaunchKernelGGL(nb_pairs_kernel<true>, dim3(nblk_pairs), dim3(tb), 0, stream, pos, mol_id, n,
                     (const GridParams*)grid, rc2, cell_start, sorted_idx, sorted_pos, sorted_mol, (int*)nullptr, row_ptr,
                     col, (int*)nullptr, (int*)nullptr, (int*)nullptr);
  hipLaunchKernelGGL(nb_sort_short_kernel, dim3(n), dim3(64), 0, stream, row_ptr, col, n);
  if (h_long > 0)
    hipLaunchKernelGGL(nb_sort_long_kernel, dim3(h_long), dim3(1024), 0, stream, row_ptr, col,
                       long_rows);
  SO2_CHECK_LAUNCH();
  return SO2_OK;
}

}  // namespace so2
