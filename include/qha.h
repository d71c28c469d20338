/*
 * qha.h -- C ABI of libqha: one GPU's share of a layer of distributed full-graph GNN training
 * with stochastically quantised halo (boundary-node) messages, for AMD MI355X (gfx950).
 *
 * The method is SYLVIE's per-layer data path (page "SYLVIE: 3D-adaptive and Universal System for
 * Large-scale Graph Neural Network Training", sections 5, 6 and 11, called "the guide" below):
 * each boundary vector is quantised at its node's bit width, sent with its (min, scale), restored
 * to float32 by the receiver and aggregated with the local rows; the backward pass does the same
 * with embedding gradients.  This library holds the device work of that path:
 *
 *   qha_quantize_pack         per-vector stochastic integer quantisation + bit packing
 *   qha_dequant_aggregate_fwd dequantisation fused into the normalised neighbour gather (SpMM)
 *                             (and an allocation-free form of it, ..._noalloc)
 *   qha_aggregate_bwd         the transposed gather that produces embedding gradients
 *   qha_aggregate_bwd_quantize the same with the halo columns' gradient rows quantised in place
 *                             (and messages received earlier added to the stored rows)
 *   qha_dense_project         the dense projection (float32 products on matrix cores) with ReLU
 *   qha_dense_backward        its gradients dA and dW in one pass (float32 products on matrix cores)
 *
 * plus small set-up helpers.  Conventions shared by every entry point:
 *   - Array arguments are caller-owned.  Pointers documented as "device" must be HIP device
 *     memory (or host memory the device can access); "host" pointers are read on the CPU.
 *   - The library allocates no memory and keeps no state between calls (the one exception is the
 *     device scratch of qha_dequant_aggregate_fwd_noalloc, declared below).  Device calls enqueue
 *     asynchronously on `stream` (a hipStream_t; NULL is the default stream) and return once
 *     the work is queued.
 *   - Every scalar and pointer argument is checked on the host before anything is enqueued; a
 *     failed check returns a status != QHA_OK and enqueues nothing.  Device data (index ranges,
 *     bits matching offsets, finite values) is a precondition: qha_validate_csr checks index
 *     arrays on the host, and kernels never read or write outside the ranges those arrays imply.
 *   - Feature rows are float32, row-major, `d` contiguous features per row, leading dimension
 *     (row stride, in elements) >= d and a multiple of 4; base pointers 16-byte aligned.
 *   - Supported widths d: 16, 32, 64, 128, 256, 512.  Index arrays are int32 (nnz < 2^31).
 *   - No exception crosses the ABI.  qha_last_error() gives a readable reason for the last
 *     failure on the calling thread.
 */
#ifndef QHA_H
#define QHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QHA_ABI_VERSION 3

/* status codes */
#define QHA_OK 0
#define QHA_ERR_INVALID_ARG 1   /* a pointer, size, stride, alignment or enum is out of contract */
#define QHA_ERR_UNSUPPORTED 2   /* well-formed but not implemented here (e.g. a width d not listed) */
#define QHA_ERR_HIP 3           /* the HIP runtime reported an error while enqueueing */
#define QHA_ERR_WORKSPACE 4     /* workspace missing or smaller than the matching *_workspace query */

/* degree normalisations for qha_degree_norm */
#define QHA_NORM_GCN 0          /* 1 / sqrt(deg + 1) */
#define QHA_NORM_MEAN 1         /* deg > 0 ? 1 / deg : 0 */

/* dense_project prologue / epilogue */
#define QHA_PRO_NONE 0
#define QHA_PRO_RELU_MASK 1     /* use a where aux > 0, else +0 (backward through ReLU) */
#define QHA_EPI_NONE 0
#define QHA_EPI_RELU 1          /* c = c > 0 ? c : +0 */

/* largest number of edges of one row that one wavefront walks (longer rows are split) */
#define QHA_DEFAULT_CHUNK 512

int qha_abi_version(void);
const char* qha_status_string(int status);
/* Reason for the most recent non-OK status returned on this thread ("" if none). */
const char* qha_last_error(void);

/* ------------------------------------------------------------------------------------------
 * Host-side set-up helpers (plain host memory, no device work)
 * ---------------------------------------------------------------------------------------- */

/* Packed-message layout (guide section 6: a b-bit integer vector per boundary node; section 9:
 * the send buffer may be grouped by width, which is only a row order).  Row r of a packed
 * buffer holds ceil(d*bits[r]/32) uint32 words (d words when bits[r] == 32, raw float32), code j
 * at bit j*bits[r], least-significant bit first.  Writes word_offset[0..n_rows] (host, exclusive
 * prefix sum, word_offset[0] = 0) and *total_words (host).  Errors: INVALID_ARG for null pointers,
 * n_rows < 0, a width not in {1,2,4,8,32}, or a total beyond 2^32-1 words; UNSUPPORTED for d. */
int qha_pack_layout(const uint8_t* bits, int64_t n_rows, int32_t d,
                    uint32_t* word_offset, uint64_t* total_words);

/* Width classes of a packed buffer whose rows are grouped by width (guide section 9: the sender
 * may group the boundary vectors it packs by bit width).  Rows start[i] .. start[i+1]-1 all have
 * width bits[i] and their codes follow each other from word base[i], so row r of class i starts
 * at base[i] + (r - start[i]) * words(d, bits[i]) with no per-row offset table: a receiver finds a
 * halo row's codes with arithmetic instead of a dependent memory load.  The layout is the same as
 * qha_pack_layout's for those rows.  Numbering the halo nodes by importance level keeps the
 * buffer grouped in every epoch, since a node's width only depends on its level and the epoch's
 * base width (guide section 9).  qha_pack_classes fills *classes from bits (host) if the rows form
 * at most QHA_MAX_CLASSES runs of equal width; otherwise it returns UNSUPPORTED and the per-row
 * word_offset/bits arrays must be used. */
#define QHA_MAX_CLASSES 8
typedef struct qha_width_classes {
  int32_t n;                             /* number of classes, 1 .. QHA_MAX_CLASSES */
  int32_t bits[QHA_MAX_CLASSES];         /* width of class i: 1, 2, 4, 8 or 32 */
  int32_t start[QHA_MAX_CLASSES + 1];    /* first row of class i; start[n] = number of rows */
  uint32_t base[QHA_MAX_CLASSES];        /* first word of class i */
} qha_width_classes;

int qha_pack_classes(const uint8_t* bits, int64_t n_rows, int32_t d, qha_width_classes* classes);

/* Checks a CSR on the host: rowptr[0] == 0, non-decreasing, rowptr[n_rows] == nnz, every
 * column in [0, n_cols), and (if require_sorted) strictly ascending columns within a row.
 * Returns QHA_OK or INVALID_ARG with the first offending row in qha_last_error(). */
int qha_validate_csr(int64_t n_rows, int64_t n_cols, const int32_t* rowptr, const int32_t* colidx,
                     int32_t require_sorted);

/* Transposes a CSR [n_rows x n_cols] into a CSR of its transpose [n_cols x n_rows] (the CSC of
 * the original): the backward pass walks the same dependencies in reverse (guide sections 3 and
 * 11), as a gather over destinations, with no atomics.  Entries of an output row come in
 * ascending original-row order.  All arrays host: colptr[n_cols+1], rowidx[nnz]. */
int qha_csr_transpose(int64_t n_rows, int64_t n_cols, const int32_t* rowptr, const int32_t* colidx,
                      int32_t* colptr, int32_t* rowidx);

/* Work plan of an aggregation over a CSR (host construction, device use).  Work is cut into items,
 * one wavefront each.  A row longer than `chunk` edges is split into chunks of at most `chunk`
 * edges, one item each; these items come first and write float64 partial sums to the workspace,
 * which a second kernel adds in chunk order (results stay deterministic).  Every other row joins a
 * group of up to QHA_GROUP_ROWS consecutive rows holding at most `group_edges` edges together (a
 * row longer than that forms a group of its own), so a wavefront streams through the contiguous
 * edge list of several short rows of a power-law graph without per-row start-up latency.  A row
 * with no edges is an item of its own, or, if skip_empty is set, belongs to no item and is left
 * as it is (valid only with beta = 1).
 * qha_agg_plan_size fills the counts; the caller allocates the device arrays, calls
 * qha_agg_plan_fill with host staging buffers of the same sizes (items: 4 * n_items int32,
 * split_row: n_split_rows, split_ptr: n_split_rows + 1), and copies them to the device.
 * qha_agg_plan_fill returns INVALID_ARG when rowptr does not give the plan's counts, and writes
 * nothing past those sizes even then. */
#define QHA_GROUP_ROWS 15
#define QHA_DEFAULT_GROUP_EDGES 256

typedef struct qha_agg_plan {
  int64_t n_rows;          /* rows of the CSR the plan was built for */
  int32_t chunk;           /* edge budget of one chunk of a split row */
  int32_t group_edges;     /* edge budget of a group of whole rows */
  int32_t skip_empty;      /* 1 if rows without edges belong to no item */
  int32_t reserved;
  int64_t n_items;         /* items */
  int64_t n_split_items;   /* leading items that are chunks of split rows (= partial-sum slots) */
  int64_t n_split_rows;    /* rows split into chunks */
  const int32_t* items;       /* device int32[4 * n_items]: first row, row count, first edge, end edge */
  const int32_t* split_row;   /* device [n_split_rows]: the split rows */
  const int32_t* split_ptr;   /* device [n_split_rows + 1]: item range of each split row */
} qha_agg_plan;

int qha_agg_plan_size(int64_t n_rows, const int32_t* rowptr, int32_t chunk, int32_t group_edges,
                      int32_t skip_empty, qha_agg_plan* plan);
int qha_agg_plan_fill(const int32_t* rowptr, const qha_agg_plan* plan, int32_t* items,
                      int32_t* split_row, int32_t* split_ptr);
/* Bytes of workspace an aggregation with this plan and width needs: one float64 partial row per
 * chunk of a split row (0 without split rows). */
size_t qha_agg_workspace_bytes(const qha_agg_plan* plan, int32_t d);

/* ------------------------------------------------------------------------------------------
 * Device entry points
 * ---------------------------------------------------------------------------------------- */

/* Degree normalisation of the GCN aggregation (guide section 2: each term is divided by
 * sqrt(d_v d_u)).  deg (device int32[n]) is a node's global degree without the self-loop
 * (section 7 asks for global, not partition-local, degree); out (device float32[n]):
 *   QHA_NORM_GCN:  1 / sqrt(deg + 1)   -- degree of A + I; the edge weight is out[v] * out[u]
 *   QHA_NORM_MEAN: deg > 0 ? 1 / deg : 0  (the GraphSAGE neighbour mean of one row)
 * Both computed with correctly rounded sqrt and division. */
int qha_degree_norm(const int32_t* deg, int64_t n, int32_t kind, float* out, void* stream);

/* Edge weights of a CSR (device): w[e] = (r ? r[i] : 1) * (c ? c[colidx[e]] : 1) in float32 for
 * every edge e of row i.  With r = c = qha_degree_norm(QHA_NORM_GCN) this is the GCN weight
 * 1/sqrt(d_v d_u) of guide section 2 as the product of the two factors; with r the mean
 * normalisation and c = NULL it is the GraphSAGE mean weight.  Set-up work, done once per graph
 * for the forward CSR and once for its transpose (where r and c swap roles). */
int qha_edge_weights(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx, const float* r,
                     const float* c, float* w, void* stream);

/* Stochastic integer quantisation and packing of message rows (guide section 6):
 *   scale = (max h - min h) / (2^b - 1), q = stochastic_round((h - min h) / scale), and the
 *   zero-point min h travels with scale; b = bits[r] in {1,2,4,8}, or 32 for a raw float32 row.
 * Row r reads x[(row_index ? row_index[r] : r) * ldx + j], j < d (device).  Its stochastic
 * rounding draws come from Philox4x32-10 with counter (node_base + r, j / 8, epoch, stream_id)
 * and key `seed`, so a call is reproducible from its arguments alone.  The row's width and the
 * start of its packed codes come from `classes` (host struct) when it is given, else from
 * bits[r] and word_offset[r] (device).  Writes the packed row (layout of qha_pack_layout) and
 * the row's metadata pair
 * meta[2r] = min (the zero-point), meta[2r + 1] = scale (device; min first, then scale, the
 * order in which they travel with the codes).
 * Floating-point steps (all float32, round-to-nearest, no contraction): mn/mx exact; zero-point
 * = mn + 0; range = mx - mn; inv = L / range; range == 0 or inv infinite -> scale 0 and codes 0;
 * else scale = range / L, y = (x - mn) * inv, q = min(floor(y) + (u16 < frac(y) * 65536), L)
 * with u16 the element's 16-bit draw.  For b = 32, codes hold the raw bits and min = scale = 0.
 * A row whose bits[r] is not in {1,2,4,8,32} is skipped (nothing written).
 * Errors: INVALID_ARG (nulls, n_rows < 0, ldx < d or not a multiple of 4, misalignment),
 * UNSUPPORTED (d), HIP.  n_rows == 0 is a no-op. */
int qha_quantize_pack(const float* x, int64_t ldx, const int32_t* row_index, int64_t n_rows,
                      int32_t d, const uint8_t* bits, const uint32_t* word_offset,
                      const qha_width_classes* classes,
                      uint64_t seed, uint32_t epoch, uint32_t stream_id, uint32_t node_base,
                      uint32_t* codes, float* meta, void* stream);

/* Dequantisation fused into the normalised neighbour aggregation (guide sections 2 and 6, the
 * receiver's "dequantize, then aggregate(local_h, remote_h)" of section 11).  For each CSR row
 * i < n_rows (device rowptr[n_rows+1], colidx[nnz]) and its output row v = row_ids ? row_ids[i] : i:
 *   out[v] = (beta ? out[v] : 0) + sum over e in row i of w[e] * x~_u,   u = colidx[e]
 *   x~_u = x_inner[u * ldx + j]                                if u < n_inner
 *        = meta[2k + 1] * q_k[j] + meta[2k]  (float32)          if u = n_inner + k, k < n_halo
 * (the raw float when the row's width is 32).  w (device float[nnz], see qha_edge_weights) may
 * be NULL for 1.0.  codes and meta are the received halo messages in qha_quantize_pack's layout;
 * each halo row's width and code offset come from `classes` (host struct) if given, else from
 * bits and word_offset (device); all may be NULL when n_halo == 0.  row_ids (device, nullable)
 * must be distinct.  plan may be NULL (one item per row); otherwise it must have been built for
 * this rowptr, and a plan with skip_empty requires beta == 1.  workspace (device, 16-byte
 * aligned) must hold qha_agg_workspace_bytes(plan, d) bytes.  beta is 0 or 1.  Each product
 * w[e] * x~_u (exact in float64) is summed in float64 in edge order (chunks of a split row
 * separately, then in chunk order), added to the old value when beta = 1 and rounded to float32
 * once; results are deterministic.  With `classes` alone (bits and word_offset NULL), x_inner's
 * rows and the packed codes must each span less than 4 GiB; otherwise the call fails with HIP
 * (invalid value) and the per-row arrays are needed.  Errors: INVALID_ARG, UNSUPPORTED (d),
 * WORKSPACE, HIP. */
int qha_dequant_aggregate_fwd(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx,
                              const float* w, const int32_t* row_ids, const qha_agg_plan* plan,
                              const float* x_inner, int64_t ldx, int64_t n_inner,
                              const uint32_t* codes, const uint32_t* word_offset,
                              const uint8_t* bits, const qha_width_classes* classes,
                              const float* meta, int64_t n_halo,
                              int32_t d, int32_t beta, float* out, int64_t ldo,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free form of qha_dequant_aggregate_fwd, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same call without the workspace arguments: the float64 partial sums of split rows go to a scratch
 * array of QHA_NOALLOC_SCRATCH_BYTES bytes that the library holds in device memory (one copy on each
 * GPU it is loaded on, kept until the process ends).  Its address is looked up once per device, on
 * the first call with that device current, after the arguments have been checked; the call then
 * allocates nothing (no hipMalloc, no library routine that allocates).  Every call on a GPU shares
 * that GPU's scratch, which keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or from several host threads) race on it and must be ordered by the caller.
 * Nothing in it needs clearing, since a call reads only partials it has written itself.
 * Errors: those of qha_dequant_aggregate_fwd; WORKSPACE when the plan's partials
 * (qha_agg_workspace_bytes) exceed QHA_NOALLOC_SCRATCH_BYTES, reported before any HIP call; HIP
 * when the scratch's device address cannot be found. */
#define QHA_NOALLOC_SCRATCH_BYTES (128u << 20)
int qha_dequant_aggregate_fwd_noalloc(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx,
                                      const float* w, const int32_t* row_ids, const qha_agg_plan* plan,
                                      const float* x_inner, int64_t ldx, int64_t n_inner,
                                      const uint32_t* codes, const uint32_t* word_offset,
                                      const uint8_t* bits, const qha_width_classes* classes,
                                      const float* meta, int64_t n_halo,
                                      int32_t d, int32_t beta, float* out, int64_t ldo, void* stream);

/* Transposed aggregation for embedding gradients (guide sections 3 and 11: gradients flow back
 * along the same cross-partition dependencies).  Given the transpose of the forward CSR
 * (qha_csr_transpose: row u lists the forward rows v that gather u) and its edge weights
 * (qha_edge_weights with the forward's r and c swapped), for u < n_rows:
 *   grad_in[u] = (beta ? grad_in[u] : 0) + sum over e in row u of w[e] * grad_out[v]
 * with v = rowidx[e] < n_grad_rows: the adjoint of qha_dequant_aggregate_fwd.  Same plan /
 * workspace / beta / precision / determinism rules.  Pass a row range [u0, u1) by offsetting
 * colptr and grad_in (w and rowidx are indexed by the absolute edge numbers in colptr). */
int qha_aggregate_bwd(int64_t n_rows, const int32_t* colptr, const int32_t* rowidx,
                      const float* w, const qha_agg_plan* plan,
                      const float* grad_out, int64_t ldg, int64_t n_grad_rows,
                      int32_t d, int32_t beta, float* grad_in, int64_t ldi,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Messages received for the stored rows of qha_aggregate_bwd_quantize (guide section 11: the
 * receiver dequantises the gradients sent back for its boundary nodes' remote copies and continues
 * backward with them added).  Stored row r gets the message rows copy_idx[copy_ptr[r] ..
 * copy_ptr[r + 1]) of this buffer, each dequantised as qha_dequant_aggregate_fwd dequantises a halo
 * row, summed in float64 in list order, added to the row's float32 value as stored without them, and
 * rounded to float32 once more: bit for bit what a following qha_dequant_aggregate_fwd with beta = 1,
 * w = NULL, n_inner = 0 and the copy lists as its CSR would leave.  The buffer must not be one the
 * call writes: these are messages that arrived before it (in the asynchronous mode of the guide's
 * section 10, the previous epoch's), which is what lets one launch both produce this epoch's
 * messages and consume earlier ones. */
typedef struct qha_received {
  const int32_t* copy_ptr;           /* device int32[n_stored + 1]: copy_ptr[0] = 0, non-decreasing */
  const int32_t* copy_idx;           /* device int32[copy_ptr[n_stored]]: message rows, each < n_rows */
  int64_t n_rows;                    /* rows of the received buffer */
  const uint32_t* codes;             /* device, qha_quantize_pack's layout */
  const float* meta;                 /* device float32[2 n_rows]: (min, scale) per row */
  const uint8_t* bits;               /* device, or NULL with classes */
  const uint32_t* word_offset;       /* device, or NULL with classes */
  const qha_width_classes* classes;  /* host, or NULL for the per-row bits / word_offset */
} qha_received;

/* The transposed gather with the sender's quantisation fused in (guide section 11: the gradients of
 * the boundary nodes are quantised with the same per-node widths and sent; section 6 for the code).
 * For every row r < n_rows of the transposed CSR it forms g_r = sum over the row's entries of
 * w * grad_out (as qha_aggregate_bwd).  Rows r < n_stored are stored, grad_in[r] = (beta ? grad_in[r]
 * : 0) + g_r, as qha_aggregate_bwd stores them; every row r >= n_stored is message row
 * m = r - n_stored, coded exactly as qha_quantize_pack codes a row holding g_r rounded to float32
 * (node id node_base + m, the same seed / epoch / stream_id, widths from classes or bits /
 * word_offset, which describe the n_rows - n_stored message rows), codes and (min, scale) written
 * in place, without storing g_r.  With n_stored = n_inner over a CSR whose rows are the inner
 * columns followed by the halo columns, one launch produces the inner nodes' embedding gradients
 * and the halo nodes' gradient messages.  Consecutive message rows of a work item share the
 * rounding generator's calls (one per lane for 512 / d rows); the draws are those of
 * qha_quantize_pack.  The plan must not skip empty rows: an empty message row is a zero gradient
 * and is coded as one.  grad_in may be NULL when n_stored = 0; codes, meta and the widths may be
 * NULL when n_stored = n_rows.  received (host struct, nullable; see qha_received) adds earlier
 * messages to the stored rows as they are written; its codes and meta must differ from this call's.
 * Arguments otherwise as in qha_aggregate_bwd and qha_quantize_pack; errors likewise. */
int qha_aggregate_bwd_quantize(int64_t n_rows, const int32_t* colptr, const int32_t* rowidx, const float* w,
                               const qha_agg_plan* plan, const float* grad_out, int64_t ldg, int64_t n_grad_rows,
                               int32_t d, int64_t n_stored, int32_t beta, float* grad_in, int64_t ldi,
                               const uint8_t* bits, const uint32_t* word_offset,
                               const qha_width_classes* classes, uint64_t seed, uint32_t epoch, uint32_t stream_id,
                               uint32_t node_base, uint32_t* codes, float* meta, const qha_received* received,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Dense projection and its gradients (guide section 2: z_v = W a_v, h_v = sigma(z_v); section 7:
 * dL/dW = sum_v (dL/dh_v * sigma'(z_v)) a_v^T), float32 products on the matrix cores (MFMA):
 *   C[m x n] = (beta ? C : 0) + op(A)[m x k] * op(B)[k x n]
 * op(X) = X (row-major, leading dimension ld) or X^T when trans_x = 1.  The forward is
 * trans_b = 1 with B = W [d_out x d_in] and epilogue RELU; the backward's dA is dZ * W and its
 * dW is dZ^T * A (trans_a = 1), both with prologue RELU_MASK and aux = the forward output H, so
 * that dZ = dH * [H > 0] is formed while A is loaded (aux has op(A)'s storage layout).
 * Each float32 operand is split exactly into three bf16 parts and each product is rebuilt on the
 * bf16 matrix cores from the six part products of weight >= 2^-16 of it (the dropped ones total
 * below 2^-23 of the product); products are accumulated in float32 over 32 values of k at a time
 * and those partial sums are added in float64; the result is rounded to float32 once (after adding
 * C when beta = 1, before the epilogue).  The error against float64 is of the size of float32
 * matrix-core products (at most 8 units of 2^-24 of sum_k |a_k b_k| per element for the
 * width-128 forward in the tests).  The width-128 forward (n = k = 128, trans_b = 1, no prologue,
 * beta = 0) runs as a row-panel kernel with W's parts held on chip; other shapes as tiled
 * products.  When m*n is small and k large the reduction is split over k
 * into float64 partials in the workspace (device, 16-byte aligned, qha_dense_project_workspace
 * bytes) and summed in a fixed order; results are deterministic.  A tiled product with
 * trans_a = 0, no split and at least 16384 rows splits B into its bf16 parts once per call when
 * the workspace holds them (qha_dense_project_workspace counts them; with less, or none, B is
 * split per tile): the same bits either way.  beta is 0 or 1.
 * Errors: INVALID_ARG, WORKSPACE (a split reduction without room for its partials), HIP. */
int qha_dense_project(int32_t trans_a, int32_t trans_b, int64_t m, int64_t n, int64_t k,
                      const float* a, int64_t lda, const float* b, int64_t ldb,
                      int32_t beta, float* c, int64_t ldc,
                      int32_t prologue, const float* aux, int64_t ld_aux, int32_t epilogue,
                      void* workspace, size_t workspace_bytes, void* stream);
size_t qha_dense_project_workspace(int32_t trans_a, int32_t trans_b, int64_t m, int64_t n, int64_t k);

/* The backward of one dense layer H = ReLU(A W^T) over m rows, in one call
 * (guide section 7: the weight gradient sums (dL/dh_v * sigma'(z_v)) a_v^T over the rows, and
 * section 3: the embedding gradient dA flows back to the aggregation):
 *   dZ = dH * [H > 0],   dA = dZ W   [m x k],   dW = dZ^T A   [n x k]
 * dH, H: device [m x n] (leading dimensions ldg, ldh); A: device [m x k] (lda); W: device [n x k]
 * (ldw); dA: device [m x k] (ldda), overwritten; dW: device [n x k] (lddw), overwritten (zeros
 * when m = 0).  Leading dimensions are multiples of 4 and at least the row width; dH, H, A and W
 * are 16-byte aligned.  dA must not overlap dH, H, A or W.  For n = k = 128 the operands are read
 * once: 32-row panels stream through on-chip memory, dZ is formed once and used for both
 * products, both products run on the bf16 matrix cores with the three-way split of
 * qha_dense_project's width-128 forward (W's parts held on chip), and per-block dW partials
 * (workspace) are added in a fixed order.  At other widths dA runs as qha_dense_project's product
 * (W split once into the workspace when it has room); dW runs by row panels when n is a multiple
 * of 128 and k of 256 (blocks of 128 x 256 outputs, each summing one range of at most about 4096
 * rows, per-range partials in the workspace), else as qha_dense_project's split product.  The
 * workspace is reused by dW after dA has read it.  dA sums are chains of 32 products accumulated
 * in float32 and added in float64; dW adds float32 sums over each block's rows in float64.  workspace: device, 16-byte aligned,
 * qha_dense_backward_workspace bytes (less only where the partials still fit).  Results are
 * deterministic.
 * Errors: INVALID_ARG, WORKSPACE, HIP. */
int qha_dense_backward(int64_t m, int64_t n, int64_t k, const float* dh, int64_t ldg, const float* h, int64_t ldh,
                       const float* a, int64_t lda, const float* w, int64_t ldw, float* da, int64_t ldda,
                       float* dw, int64_t lddw, void* workspace, size_t workspace_bytes, void* stream);
size_t qha_dense_backward_workspace(int64_t m, int64_t n, int64_t k);

/* ------------------------------------------------------------------------------------------
 * Host-side width control (plain host memory, no device work)
 * ---------------------------------------------------------------------------------------- */

/* Graph Extractor (guide section 7).  deg: host [n] global in-degrees of the boundary-node pool.
 * A node's importance is the fraction of the pool whose degree is at most its own (the largest
 * degree gets 1, equal degrees equal importance, relabelling nodes changes nothing); with
 * n_levels candidate widths its mask level is ceil(importance * n_levels) - 1, computed exactly
 * in integers.  Writes level (host [n]) and, if not NULL, importance (host [n]).
 * Errors: INVALID_ARG (null arrays, n < 0, n_levels outside 1 .. QHA_MAX_LEVELS). */
#define QHA_MAX_LEVELS 8
int qha_mask_levels(const int32_t* deg, int64_t n, int32_t n_levels, uint8_t* level, double* importance);

/* Quant Orchestrator (guide section 9, Figure 7): the epoch's per-node widths from the mask
 * levels and the Coordinator's base width, bits[i] = min(base_bits << level[i], max_bits).
 * base_bits and max_bits are 1, 2, 4 or 8, base_bits <= max_bits; levels < QHA_MAX_LEVELS.
 * Host arrays.  Errors: INVALID_ARG. */
int qha_node_bits(const uint8_t* level, int64_t n, int32_t base_bits, int32_t max_bits, uint8_t* bits);

/* A halo numbering by descending mask level (ties keep their order): order[i] is the node placed
 * at position i.  Widths from qha_node_bits never increase along it, for every base width, so a
 * buffer packed in this order stays grouped by width (qha_pack_classes) in every epoch.
 * Host arrays.  Errors: INVALID_ARG. */
int qha_level_order(const uint8_t* level, int64_t n, int32_t* order);

/* Coordinator (guide section 8, Eq. 3-5).  One call per epoch t with the partitions' losses and
 * the epoch's time: L_t = mean loss, F_t = lambda F_{t-1} + (1 - lambda) L_t (F starts at L_0),
 * LDR_t = (F_t - F_{t-1}) / time.  The returned base width for epoch t + 1 is b_min after epoch 0;
 * for t > delta it doubles (at most b_max) if LDR_t < LDR_{t-delta} and halves (at least b_min)
 * otherwise, with the next epoch synchronous in the first case and asynchronous in the second;
 * for 0 < t <= delta width and mode stay.  descent_magnitude = 1 compares -LDR instead (the
 * reading where "LDR got worse" means the descent slowed).  The state is caller-owned and plain
 * data.  Errors: INVALID_ARG (lambda outside [0, 1], delta outside 1 .. QHA_LDR_MAX_DELTA, widths
 * not powers of two in 1 .. 8 with b_min <= b_max, no partitions, a non-positive time). */
#define QHA_LDR_MAX_DELTA 64
typedef struct qha_coordinator {
  double lambda;
  double sign;                           /* +1, or -1 with descent_magnitude */
  double f_prev;                         /* F_{t-1} */
  double last_ldr;                       /* LDR of the last recorded epoch */
  double ldr[QHA_LDR_MAX_DELTA + 1];     /* the last delta + 1 LDR values, by t % (delta + 1) */
  int64_t t;                             /* epochs recorded so far */
  int32_t delta, b_min, b_max;
  int32_t bits;                          /* base width of the next epoch */
  int32_t sync;                          /* 1: the next epoch runs synchronously */
} qha_coordinator;

int qha_coordinator_init(qha_coordinator* c, double lambda, int32_t delta, int32_t b_min, int32_t b_max,
                         int32_t descent_magnitude);
int qha_coordinator_step(qha_coordinator* c, const double* losses, int32_t n_partitions, double epoch_time,
                         int32_t* next_bits, int32_t* next_sync);

#ifdef __cplusplus
}
#endif
#endif /* QHA_H */
