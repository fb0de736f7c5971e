/*
 * so2attn.h - C ABI of the MI355X (gfx950) on-the-fly SO(2) equivariant
 * graph attention forward pass.
 *
 * The operation (stated in prose, without equations, by "E2Former-V2:
 * On-the-Fly Equivariant Attention with Linear Activation Memory",
 * technical summary, sections 2.1 and 2.2; envelope placement from
 * "EquiformerV3: Scaling Efficient, Expressive, and General SE(3)-Equivariant
 * Graph Attention Transformers", technical summary, section 2.B.3):
 *
 *   For every target atom i, stream its neighbours j within the cutoff.
 *   For each edge, rotate the neighbour's irreps features x_j into the frame
 *   whose z axis is the edge vector, gate them per channel with a radial
 *   function of the edge length, apply one linear map per |m| (real for
 *   m = 0, complex W1 + i W2 for m >= 1, mixing all degrees l >= |m| and all
 *   channels), rotate the result back.  Weight the messages with a softmax
 *   over j of the invariant logits q_i . k_j / sqrt(d) per head, multiplied
 *   by a smooth cutoff envelope in numerator and denominator, and sum them.
 *   No per-edge tensor is written to device memory.
 *
 * Layouts
 *   irreps component index of (l, m): l*l + l + m, m = -l..l; real
 *   spherical harmonics with z as polar axis and no Condon-Shortley phase
 *   (l = 1 components are the (y, z, x) parts of a vector).
 *   x       [n_atoms][(L+1)^2][C]    in `dtype`
 *   y       [n_targets][(L+1)^2][C]  fp32 (always)
 *   w_q,w_k [C][C] as (in, out): q_i[o] = sum_c x_i[0][c] w_q[c][o]
 *   w_rad   [K][C]: g_ij[c] = sum_k phi_k(|r_ij|) w_rad[k][c], Gaussian
 *           phi_k with centres k*rc/(K-1) and width rc/(K-1)
 *   w_so2   packed: W0 [(L+1)C][(L+1)C], then for m = 1..L the pair
 *           W1_m, W2_m, each [(L+1-m)C][(L+1-m)C]; every block row-major
 *           [out][in] with row/column index (l - m)*C + c
 *   head h owns channels [h*C/H, (h+1)*C/H)
 *   edge vector r_ij = p_j - p_i (target i, source j), minimum image when a
 *   box is given; envelope u(s) = 1 - (p+1)(p+2)/2 s^p + p(p+2) s^(p+1)
 *   - p(p+1)/2 s^(p+2) for s = |r_ij|/rc < 1, else 0.
 *
 * Conventions for every call
 *   Pointers are device pointers unless the name ends in _host.  The caller
 *   owns every buffer; the library allocates no device memory: scratch comes
 *   from the caller's `workspace` (size from the *_workspace_bytes query,
 *   256-byte alignment required).  Argument errors are detected on the host
 *   before anything is launched and leave every output untouched.  Calls on
 *   different streams may run concurrently if their buffers do not overlap.
 *   `stream` is a hipStream_t (NULL = the default stream).
 */
#ifndef SO2ATTN_H
#define SO2ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* so2_stream_t; /* same object as hipStream_t */

typedef enum {
  SO2_OK = 0,
  SO2_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, non-finite position */
  SO2_ERR_UNSUPPORTED = 2,      /* legal shape with no kernel (e.g. C > 256)   */
  SO2_ERR_CAPACITY = 3,         /* col[] too small; *n_edges_host = required E */
  SO2_ERR_BOX = 4,              /* a box side <= 2 * cutoff                    */
  SO2_ERR_DEVICE = 5,           /* a HIP call failed                            */
  SO2_ERR_WORKSPACE = 6         /* workspace too small or misaligned            */
} so2_status;

typedef enum { SO2_FP32 = 0, SO2_BF16 = 1 } so2_dtype;

enum {
  SO2_FLAG_RBF_ENVELOPE = 1u, /* alternative reading: phi_k is also multiplied by u */
  SO2_FLAG_NO_RADIAL = 2u     /* g_ij == 1 (special-case tests)                      */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* so2_status_string(so2_status status);

/* Text of the last HIP error seen by this thread inside the library, or "". */
const char* so2_last_device_error(void);

/* ------------------------------------------------------------------------
 * build_neighbors - radius graph N(i) = { j != i : same molecule,
 *   |mic(p_j - p_i)| < cutoff } as CSR with j ascending in every row.
 * Follows the neighbour set the E2Former-V2 summary streams over (technical
 * section 2.2).  The boundary test is done in fp64 with this exact operation
 * sequence, so the result is bit-identical to a brute-force search that does
 * the same: dx = (double)pj.x - (double)pi.x; with a box side b,
 * dx = dx - b * rint(dx / b) (ties to even); s = (dx*dx + dy*dy) + dz*dz,
 * each operation rounded separately; keep iff s < (double)cutoff^2.
 *
 *   pos          [n_atoms][3] fp32 (device)
 *   mol_id       [n_atoms] int32 (device) or NULL: pairs in different
 *                molecules are never neighbours
 *   box_host     float[3] orthorhombic periodic box (host) or NULL (open)
 *   row_ptr      [n_atoms+1] int32 (device, written)
 *   col          [capacity] int32 (device, written)
 *   n_edges_host out: E = row_ptr[n_atoms]; on SO2_ERR_CAPACITY the number
 *                of entries col[] needs (row_ptr is then written, col not)
 *   workspace    >= so2_neighbors_workspace_bytes(n_atoms) bytes (device)
 * Errors: INVALID_ARGUMENT (nulls, n_atoms < 1, cutoff <= 0 or not finite,
 * non-finite positions, E > INT32_MAX), BOX (side <= 2*cutoff), CAPACITY,
 * WORKSPACE, DEVICE.
 * Synchronisation: the call waits for `stream` once, for E (the bounding box
 * and the cell grid are computed on the device), and returns once E is
 * known; the fill and the row sort are left queued on `stream`.  Non-finite
 * positions are reported at that point, before the fill.  Cost O(N) memory, O(N k) work.
 * ---------------------------------------------------------------------- */
size_t so2_neighbors_workspace_bytes(int32_t n_atoms);

so2_status build_neighbors(const float* pos, int32_t n_atoms, const int32_t* mol_id,
                           const float* box_host, float cutoff, int32_t* row_ptr,
                           int32_t* col, int64_t capacity, int64_t* n_edges_host,
                           void* workspace, size_t workspace_bytes, so2_stream_t stream);

/* ------------------------------------------------------------------------
 * so2_attention_fwd - the fused forward pass described at the top.
 * Follows the E2Former-V2 summary (technical sections 2.1, 2.2): query and
 * key are projections of the invariant l = 0 slice, the softmax over N(i)
 * is gated by the envelope in numerator and denominator ("EquiformerV3: ...", technical summary, section 2.B.3), y_i = 0 when N(i) is empty.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_atoms;    /* rows of x and pos                                    */
  int32_t n_targets;  /* outputs y[0..n_targets) (targets are atoms 0..T-1)   */
  int64_t n_edges;    /* >= row_ptr[n_targets] - row_ptr[0]; sizes workspace  */
  int32_t l_max;      /* 0..6                                                 */
  int32_t channels;   /* C >= 1                                               */
  int32_t heads;      /* H >= 1, C % H == 0                                   */
  int32_t n_rbf;      /* K >= 2                                               */
  int32_t envelope_p; /* envelope exponent p >= 1 (5 in the usual setting)    */
  float cutoff;       /* rc > 0, the same value build_neighbors used          */
  uint32_t flags;     /* SO2_FLAG_*                                           */
  int32_t dtype;      /* so2_dtype of x and of every weight                   */
} so2_attn_desc;

/* Number of w_so2 entries: C^2 [(L+1)^2 + L(L+1)(2L+1)/3]; -1 on bad input. */
int64_t so2_weight_count(int32_t l_max, int32_t channels);

/* Workspace so2_attention_fwd needs (0 if desc is invalid). */
size_t so2_attention_workspace_bytes(const so2_attn_desc* desc);

/* Which kernel so2_attention_fwd runs for desc: 0 = none (unsupported),
 * 1 = fp32 VALU kernel, 2 = bf16 MFMA kernel. */
int32_t so2_attention_kernel_kind(const so2_attn_desc* desc);

/*   desc      host struct above
 *   pos       [n_atoms][3] fp32; box_host float[3] or NULL, as for the graph
 *   row_ptr   [n_atoms+1], col [E]: the CSR from build_neighbors (rows
 *             0..n_targets-1 are read)
 *   x         [n_atoms][(L+1)^2][C]          dtype
 *   w_q, w_k  [C][C], w_rad [K][C], w_so2 [so2_weight_count]   dtype
 *   y         [n_targets][(L+1)^2][C] fp32, written
 *   workspace >= so2_attention_workspace_bytes(desc) bytes
 * Kernels: bf16 with C = 128, 1 <= L <= 6, H <= 16, K <= 32 runs on the
 * MFMA kernel; every other shape (fp32 or bf16) on the VALU kernel.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (L > 6 or C > 256: no kernel), BOX,
 * WORKSPACE, DEVICE.  Asynchronous on
 * `stream`.  Device memory beyond the caller's buffers: none; activation
 * memory is O(n_atoms) (workspace), never O(E). */
so2_status so2_attention_fwd(const so2_attn_desc* desc, const float* pos,
                             const float* box_host, const int32_t* row_ptr,
                             const int32_t* col, const void* x, const void* w_q,
                             const void* w_k, const void* w_rad, const void* w_so2,
                             float* y, void* workspace, size_t workspace_bytes,
                             so2_stream_t stream);

/* Benchmark hook: when both are non-NULL, every later so2_attention_fwd
 * call from this thread records `start` on its stream just before the fused
 * attention kernel and `stop` just after it, and every later so2_swiglu_s2
 * call does the same around its grid kernel (hipEvent_t handles created and
 * owned by the caller), so the kernel alone can be timed on the stream it
 * runs on.  so2_set_kernel_timing_events(NULL, NULL) switches it off. */
void so2_set_kernel_timing_events(void* start, void* stop);

/* ------------------------------------------------------------------------
 * so2_merged_rms_norm - equivariant merged RMS layer norm of node features
 * ("EquiformerV3: Scaling Efficient, Expressive, and General SE(3)-Equivariant
 * Graph Attention Transformers", technical summary, section 2.B.1: one RMS
 * statistic shared by all degrees of a node):
 *   y[i][(l,m)][c] = gamma[l][c] x[i][(l,m)][c] / sqrt(mean_{l,m,c} x[i]^2 + eps)
 *   x        [n_atoms][(l_max+1)^2][channels] dtype (device)
 *   gamma    [l_max+1][channels] fp32 (device): gain per degree and channel
 *   y        same shape and dtype as x (device); may be x itself (in place)
 *   eps      >= 0, finite
 * Statistics in fp32; bf16 outputs are rounded to nearest even.
 * Errors: INVALID_ARGUMENT (nulls with n_atoms > 0, n_atoms < 0, l_max < 0,
 * channels < 1, bad eps or dtype), UNSUPPORTED (l_max > 6), DEVICE.
 * Asynchronous on `stream`; no workspace, no device allocation.
 * ---------------------------------------------------------------------- */
so2_status so2_merged_rms_norm(const void* x, const float* gamma, void* y, int32_t n_atoms, int32_t l_max,
                               int32_t channels, float eps, int32_t dtype, so2_stream_t stream);

/* ------------------------------------------------------------------------
 * so2_swiglu_s2 - SwiGLU-S2 activation of node features ("EquiformerV3:
 * Scaling Efficient, Expressive, and General SE(3)-Equivariant Graph
 * Attention Transformers", technical summary, section 2.C: features on a
 * sphere grid, the nonlinear gate on the scalar channels only, a bilinear
 * product of grid features).  Per node, with Y the real harmonics:
 *   u = x A_l, v = x B_l            (per degree l, row vectors of C channels)
 *   g = x[(0,0)] G
 *   h[(l,m)] = sum_p w_p Y_lm(r_p) u(r_p) v(r_p)    for l <= l_max
 *   y[(l,m)] = (SiLU(g) * h[(l,m)]) O_l
 * on the product grid of ceil((3 l_max + 1) / 2) Gauss-Legendre nodes in
 * cos(theta) times 3 l_max + 1 equally spaced phi (exact for the degree
 * <= 3 l_max integrands, so the map is equivariant).
 *   x              [n_atoms][(l_max+1)^2][channels] dtype (device)
 *   w_a, w_b, w_o  [l_max+1][channels][channels] dtype, [l][in][out] (device)
 *   w_g            [channels][channels] dtype, [in][out] (device)
 *   y              [n_atoms][(l_max+1)^2][channels] fp32, written (device)
 *   workspace      >= so2_swiglu_s2_workspace_bytes(...) bytes, 16-byte
 *                  aligned (device): u, v, g and the gated product
 * bf16 with channels = 128 and 16-byte aligned x and weights runs the maps on
 * the matrix cores (bf16 operands, fp32 sums) and keeps u, v and the gated
 * product in bf16; every other shape runs in fp32 arithmetic.
 * Errors: INVALID_ARGUMENT (nulls with n_atoms > 0, n_atoms < 0, l_max < 0,
 * channels < 1, bad dtype), UNSUPPORTED (l_max > 6), WORKSPACE, DEVICE.
 * Asynchronous on `stream`; no device allocation.  The workspace query
 * returns 0 for arguments the call rejects.
 * ---------------------------------------------------------------------- */
size_t so2_swiglu_s2_workspace_bytes(int32_t n_atoms, int32_t l_max, int32_t channels, int32_t dtype);
so2_status so2_swiglu_s2(const void* x, const void* w_a, const void* w_b, const void* w_g, const void* w_o, float* y,
                         int32_t n_atoms, int32_t l_max, int32_t channels, int32_t dtype, void* workspace,
                         size_t workspace_bytes, so2_stream_t stream);

/* ------------------------------------------------------------------------
 * Host-side diagnostics (no device work): evaluate, on the CPU, the same
 * edge-frame and Wigner-D code the kernels run in fp32, for tests.
 *   rhat   float[3] edge direction (need not be normalised)
 *   R_out  float[9] row-major rotation with R rhat = z_hat (the kernels' gauge)
 *   D_out  float[sum_{l<=L} (2l+1)^2]: blocks D^0..D^L, each row-major with
 *          rows/cols m = -l..l, such that Y_l(R s) = D^l Y_l(s)
 * Returns INVALID_ARGUMENT for nulls, a zero vector or L outside 0..6.
 * ---------------------------------------------------------------------- */
so2_status so2_edge_frame_host(int32_t l_max, const float* rhat, float* R_out, float* D_out);

#ifdef __cplusplus
}
#endif

#endif /* SO2ATTN_H */
