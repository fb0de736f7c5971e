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
 *   - p(p+1)/2 s^(p+2) for s = |r_ij|/rc < 1, else 0, evaluated as
 *   (1-s)^3 sum_{k<p} (k+1)(k+2)/2 s^k with |r_ij| and 1-s in fp64, so it
 *   keeps its relative precision for edges just inside the cutoff.
 *
 * Conventions for every call
 *   Pointers are device pointers unless the name ends in _host.  The caller
 *   owns every buffer; the library allocates no device memory and creates no
 *   streams or events: scratch comes from the caller's `workspace` (size
 *   from the *_workspace_bytes query, 256-byte alignment required), and
 *   every kernel runs on the caller's `stream` (a hipStream_t, NULL = the
 *   default stream).  Calls keep no state between them (apart from the text
 *   behind so2_last_device_error, which is per host thread), so they are
 *   thread-safe; calls on different streams may run concurrently if their
 *   buffers, workspaces included, do not overlap.  Argument errors are
 *   detected on the host before anything is launched and leave every output
 *   untouched.
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

/* Steps of so2_attention_fwd, for so2_attention_fwd_stages. */
enum {
  SO2_STAGE_PREPARE = 1u, /* q/k projection and the fused kernel's prologue (workspace) */
  SO2_STAGE_FUSED = 2u    /* the fused attention kernel: workspace -> y               */
};

/* Steps of so2_swiglu_s2, for so2_swiglu_s2_stages. */
enum {
  SO2_STAGE_SW_MAPS = 1u, /* per-degree maps u, v and the gate map g (workspace) */
  SO2_STAGE_SW_GRID = 2u, /* grid product and gate (workspace -> workspace)      */
  SO2_STAGE_SW_OUT = 4u   /* per-degree output maps (workspace -> y)             */
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

/* Which path so2_attention_fwd runs for desc: 0 = none (the call returns
 * UNSUPPORTED), 2 = bf16 MFMA kernel, 3 = fp32 edge-batch path (1, the fp32
 * VALU kernel, is what so2_attention_fwd_noalloc takes instead of 3). */
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
 * MFMA kernel (bf16 operands, fp32 accumulation); that kernel needs x, w_rad
 * and w_so2 16-byte aligned (else INVALID_ARGUMENT) and addresses its
 * repacked copy of x with 32-bit offsets, which caps n_atoms at
 * (2^32 - 2^16) / (2 (L+1)(L+2) C) (about 559k atoms at L = 4, 299k at
 * L = 6); beyond that the call returns UNSUPPORTED.  Every other shape
 * (fp32, or bf16 with other C, L, H or K) runs on the fp32 edge-batch path:
 * per-edge kernels for the frame, the rotations and the softmax weights,
 * the per-m maps as fp32 GEMMs on the matrix cores over batches of 64 edges
 * per target (4096 to 65536 edges, fixed by n_targets), and a per-target
 * sum in edge order (bitwise repeatable).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (L > 6, C > 256, H > 256, or the
 * MFMA shape past its atom limit), BOX, WORKSPACE, DEVICE.
 * Stream: the MFMA kernel is asynchronous on `stream`; the edge-batch path
 * reads row_ptr[0] and row_ptr[n_targets] back to plan its batches, which
 * waits on `stream` once.
 * Device memory beyond the caller's buffers: none; activation memory is
 * O(n_atoms) (workspace; the edge-batch path adds one batch of per-edge
 * tensors, a constant), never O(E). */
so2_status so2_attention_fwd(const so2_attn_desc* desc, const float* pos,
                             const float* box_host, const int32_t* row_ptr,
                             const int32_t* col, const void* x, const void* w_q,
                             const void* w_k, const void* w_rad, const void* w_so2,
                             float* y, void* workspace, size_t workspace_bytes,
                             so2_stream_t stream);

/* so2_attention_fwd in steps: `stages` is SO2_STAGE_PREPARE, SO2_STAGE_FUSED
 * or both (both = so2_attention_fwd).  PREPARE writes the query/key
 * projections, the softmax statistics, the repacked operands and the run
 * schedule into the workspace; FUSED reads them and writes y.  A FUSED call
 * must follow a PREPARE call with the same arguments and workspace, on the
 * same stream or ordered after it; y may be NULL for PREPARE alone.  The
 * split lets a caller time the fused kernel by itself or overlap the
 * prologue with other work.  Same errors as so2_attention_fwd, plus
 * INVALID_ARGUMENT for an empty or unknown `stages`. */
so2_status so2_attention_fwd_stages(uint32_t stages, const so2_attn_desc* desc, const float* pos,
                                    const float* box_host, const int32_t* row_ptr, const int32_t* col,
                                    const void* x, const void* w_q, const void* w_k, const void* w_rad,
                                    const void* w_so2, float* y, void* workspace, size_t workspace_bytes,
                                    so2_stream_t stream);

/* ------------------------------------------------------------------------
 * so2_attention_fwd_variant - the forward with variants of the value path
 * and the logits.  "DPA4: Pushing the Accuracy-Cost Frontier of
 * Interatomic Potentials with EMFA SO(2) Convolution", technical summary,
 * section 2.1 A2: the hidden channels split into F focus streams, each with
 * its own SO(2) stack, reweighted per edge by a softmax across streams from
 * the invariant l = 0 section.  Per edge, in the edge frame:
 *   m_max      the per-m maps stop at |m| = m_max (rows above give 0)
 *   w_logit    [K][H] in dtype, or NULL: z_ij^h += sum_k phi_k(|r_ij|)
 *              w_logit[k][h] (the gate's Gaussian basis, no envelope)
 *   n_focus F  channels [f C/F, (f+1) C/F) form stream f; w_so2 is F stacks
 *              back to back, stack f the packing above over C/F channels
 *              (so2_weight_count_variant entries in all); stream f of the
 *              edge message is scaled by pi_f = softmax_f(sum_{c in f}
 *              w_focus[c] yt[(0,0), c])
 *   w_focus    [C] in dtype, required when n_focus > 1
 * Kernels (so2_attention_variant_kernel_kind says which): bf16 MFMA shapes
 * run on the MFMA kernel with one stream and any m_max (the instance of
 * that m_max has no passes for |m| > m_max), and with F = 2, 4 or 8 streams
 * at l_max <= 4, every order, F dividing heads (block-diagonal weights, the
 * cross-focus softmax from a score pass over the m = 0 chunks); every other
 * variant and shape runs on the fp32 edge-batch path.  Other
 * arguments, the workspace (so2_attention_variant_workspace_bytes) and the
 * errors are those of so2_attention_fwd, plus INVALID_ARGUMENT for m_max
 * outside -1..l_max, n_focus < 1 or not dividing C, or a missing w_focus.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t m_max;   /* orders |m| <= m_max; -1 = l_max (every order)      */
  int32_t n_focus; /* F >= 1 focus streams of C / F channels (1 = one)   */
} so2_attn_variant;

/* Entries of w_so2 for a variant: F C'^2 [(L+1)^2 + 2 sum_{m=1..m_max}
 * (L+1-m)^2], C' = C / F; -1 on bad input. */
int64_t so2_weight_count_variant(int32_t l_max, int32_t channels, int32_t m_max, int32_t n_focus);
size_t so2_attention_variant_workspace_bytes(const so2_attn_desc* desc, const so2_attn_variant* var);
int32_t so2_attention_variant_kernel_kind(const so2_attn_desc* desc, const so2_attn_variant* var);
so2_status so2_attention_fwd_variant(const so2_attn_desc* desc, const so2_attn_variant* var, const float* pos,
                                     const float* box_host, const int32_t* row_ptr, const int32_t* col,
                                     const void* x, const void* w_q, const void* w_k, const void* w_rad,
                                     const void* w_so2, const void* w_logit, const void* w_focus, float* y,
                                     void* workspace, size_t workspace_bytes, so2_stream_t stream);

/* ------------------------------------------------------------------------
 * so2_attention_bwd - gradients of a scalar loss L through so2_attention_fwd,
 * for forces and training ("E2Former-V2: On-the-Fly Equivariant Attention
 * with Linear Activation Memory", technical summary, section 4: the
 * Conservative variant takes forces as derivatives of the energy through
 * the layer; "DPA4: Pushing the Accuracy-Cost Frontier of Interatomic
 * Potentials with EMFA SO(2) Convolution", technical summary, section 2.2:
 * conservative training differentiates the energy-to-force path).  Given
 * dy = dL/dy, returns dL/dx, dL/dpos and dL/dW for the same forward (same
 * descriptor, graph and inputs).  Memory stays linear in the atom count:
 * per-edge tensors exist only for one batch of edges at a time (64 per
 * target, between 4096 and 65536 edges, fixed by n_targets), and only the
 * softmax statistics and head sums per (target, head) live across batches.
 *   dy        [n_targets][(L+1)^2][C] fp32
 *   dx        [n_atoms][(L+1)^2][C] fp32, written (sources and targets)
 *   dpos      [n_atoms][3] fp32, written; minus the forces when L is an
 *             energy.  Row sums are zero up to rounding (translation
 *             invariance).
 *   dw_q, dw_k [C][C], dw_rad [K][C], dw_so2 [so2_weight_count] fp32,
 *             written; each may be NULL (not computed: the force-only path
 *             skips the weight reductions)
 *   workspace >= so2_attention_bwd_workspace_bytes(desc) bytes
 * Arithmetic: fp32, except the three uses of the per-m map (the forward
 * map recomputed, its transpose, the weight gradient), GEMMs over each
 * batch on the matrix cores: fp32 GEMMs for fp32 inputs; for bf16 inputs
 * bf16-operand GEMMs with fp32 accumulation, each fp32 operand split into
 * two bf16 parts hi + lo (about 16 significant bits; the weight matrices
 * are exact in bf16 and not split).  Measured errors against the fp64
 * oracle: about 1e-6 (fp32 inputs), 5e-6 to 3e-4 (bf16 inputs; the bound is
 * the bf16 one, 2e-2).  Contributions to dx of sources, dpos, dq, dk and
 * the weights are summed with fp32 atomics, so the low bits vary between
 * runs.
 * Shapes: L <= 6, C <= 256, H <= 256, else UNSUPPORTED.  A target whose
 * envelopes are all 0 (edges exactly at the cutoff only) has y = 0 and
 * gets no gradient.
 * Errors: INVALID_ARGUMENT (also row_ptr[n_targets] < row_ptr[0]),
 * UNSUPPORTED, BOX, WORKSPACE, DEVICE.
 * Stream: the call reads row_ptr[0] and row_ptr[n_targets] back to the host
 * to plan its batches, which synchronises `stream` once; everything else is
 * enqueued on `stream`.  No device allocation.
 * ---------------------------------------------------------------------- */
size_t so2_attention_bwd_workspace_bytes(const so2_attn_desc* desc);
so2_status so2_attention_bwd(const so2_attn_desc* desc, const float* pos, const float* box_host,
                             const int32_t* row_ptr, const int32_t* col, const void* x, const void* w_q,
                             const void* w_k, const void* w_rad, const void* w_so2, const float* dy, float* dx,
                             float* dpos, float* dw_q, float* dw_k, float* dw_rad, float* dw_so2, void* workspace,
                             size_t workspace_bytes, so2_stream_t stream);

/* ------------------------------------------------------------------------
 * so2_attention_fwd_noalloc - so2_attention_fwd for callers that cannot
 * allocate device memory: code under stream (HIP graph) capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments and results
 * as so2_attention_fwd without the workspace: the call uses a device array
 * of SO2_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends (looked up once per device on the first call
 * there), and it allocates nothing and never waits on the stream: shapes
 * that so2_attention_fwd runs on the edge-batch path run here on the fp32
 * VALU kernel (one workgroup per target, asynchronous).  The caller still
 * passes inputs and y.
 *   Limit: the workspace of that kernel <= SO2_NOALLOC_SCRATCH_BYTES
 *   (about 14,000 atoms at L = 4, C = 128, bf16; 8,500 at L = 6), else
 *   SO2_ERR_WORKSPACE before anything is launched.
 *   Every call rewrites all of the array it reads, so nothing carries over
 *   from an earlier call; but calls on one GPU share the array: calls that
 *   overlap in time on that GPU (different streams or host threads) race
 *   and must be serialised by the caller.
 * Errors: those of so2_attention_fwd; WORKSPACE past the limit.
 * ---------------------------------------------------------------------- */
#define SO2_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

so2_status so2_attention_fwd_noalloc(const so2_attn_desc* desc, const float* pos, const float* box_host,
                                     const int32_t* row_ptr, const int32_t* col, const void* x,
                                     const void* w_q, const void* w_k, const void* w_rad,
                                     const void* w_so2, float* y, so2_stream_t stream);

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
 *                  aligned (device): u, v, g and the gated product, or the
 *                  weights repacked for the fused kernel (under 0.6 MB)
 * bf16 with channels = 128 and 16-byte aligned x and weights runs the maps on
 * the matrix cores (bf16 operands, fp32 sums) and keeps u, v and the gated
 * product in bf16; at l_max <= 4 the whole call is one fused kernel (groups
 * of 4 nodes through maps, grid and output map in LDS), whose results are
 * bitwise those of the three steps of so2_swiglu_s2_stages.  Every other
 * shape runs in fp32 arithmetic.
 * Errors: INVALID_ARGUMENT (nulls with n_atoms > 0, n_atoms < 0, l_max < 0,
 * channels < 1, bad dtype), UNSUPPORTED (l_max > 6), WORKSPACE, DEVICE.
 * Asynchronous on `stream`; no device allocation.  The workspace query
 * returns 0 for arguments the call rejects.
 * ---------------------------------------------------------------------- */
size_t so2_swiglu_s2_workspace_bytes(int32_t n_atoms, int32_t l_max, int32_t channels, int32_t dtype);
so2_status so2_swiglu_s2(const void* x, const void* w_a, const void* w_b, const void* w_g, const void* w_o, float* y,
                         int32_t n_atoms, int32_t l_max, int32_t channels, int32_t dtype, void* workspace,
                         size_t workspace_bytes, so2_stream_t stream);

/* so2_swiglu_s2 in steps: `stages` is any non-empty union of
 * SO2_STAGE_SW_MAPS, SO2_STAGE_SW_GRID and SO2_STAGE_SW_OUT (all three =
 * so2_swiglu_s2); the steps run in that order and pass their results
 * through the workspace, so a step must follow the earlier ones with the same
 * arguments and workspace, on the same stream or ordered after them.  Lets a
 * caller time or overlap the steps.  Same errors as so2_swiglu_s2, plus
 * INVALID_ARGUMENT for an empty or unknown `stages`. */
so2_status so2_swiglu_s2_stages(uint32_t stages, const void* x, const void* w_a, const void* w_b, const void* w_g,
                                const void* w_o, float* y, int32_t n_atoms, int32_t l_max, int32_t channels,
                                int32_t dtype, void* workspace, size_t workspace_bytes, so2_stream_t stream);

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

/* The rotation generators the backward uses, on the CPU by the same code:
 * J_out[a * N + ...] (N = sum_{l<=L} (2l+1)^2, a = x, y, z) holds the blocks
 * of d/dt D^l(exp(t [e_a]x)) at t = 0 for l = 0..L, each row-major like
 * so2_edge_frame_host's D.  INVALID_ARGUMENT for a null pointer or L
 * outside 0..6. */
so2_status so2_wigner_generators_host(int32_t l_max, float* J_out);

#ifdef __cplusplus
}
#endif

#endif /* SO2ATTN_H */
