/*
 * embcore.h -- C ABI of the MI355X (gfx950) sparse-embedding + dot-interaction core.
 *
 * The calls follow the model statement of the page "DLRM For PyTorch" (§Model
 * architecture): dense features go through a bottom MLP, every categorical feature has its
 * own embedding table, the bottom-MLP output and the embedding vectors meet in a "dot
 * interaction" whose output is concatenated with the bottom-MLP output and fed to the top
 * MLP.  This library holds the part between the MLPs: the embedding-bag gather, the
 * interaction forward and backward, and the sparse SGD update of the embedding rows.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns all memory; the
 *     library allocates nothing and keeps no state between calls, except the static
 *     scratch array of emb_grad_reduce_update_noalloc (one per GPU, see there).
 *   - Work is enqueued on `stream` and runs asynchronously; no call synchronises.
 *   - Arguments are validated on the host before anything is enqueued.  A call that
 *     returns a status other than EL_OK has enqueued nothing, except EL_ERR_HIP, which
 *     reports a launch failure (text from el_last_error()).
 *   - Outputs must not alias inputs.  Only emb_grad_reduce_update writes to the tables.
 *   - Every call with the same inputs produces bitwise identical outputs: no call adds
 *     floating-point values with atomics.  The integer atomics that remain (the radix
 *     sort's LDS digit counters, el_validate_bags' defect count) give exact counts in any
 *     order.
 *   - Float conversions round to nearest even; denormals are kept; NaN stays NaN.
 */
#ifndef EMBCORE_H
#define EMBCORE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define EL_API __attribute__((visibility("default")))
#else
#define EL_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EL_OK = 0,
  EL_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size, inconsistent shape */
  EL_ERR_UNSUPPORTED = 2, /* valid request the library does not implement (e.g. row size) */
  EL_ERR_WORKSPACE = 3,   /* workspace smaller than emb_grad_workspace_bytes() */
  EL_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} el_status;

typedef enum {
  EL_F32 = 0,
  EL_F16 = 1,
  EL_BF16 = 2,
  /* Not dtypes.  With these two bounds every int32 is a value of the type, so an unknown
   * code that a caller passes (from C, Python, ...) reaches the checks, which refuse it,
   * instead of being an out-of-range enum value in the library's C++. */
  EL_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  EL_DTYPE_RANGE_MAX_ = 2147483647
} el_dtype;

/* --hash_indices (page "DLRM For PyTorch", §Command-line options): replace every index by
 * index mod table size, with the floor-modulo sign convention (a negative index maps into
 * the table).  Without the flag an index outside [0, rows of its table) is undefined
 * behaviour in the gather/update calls; el_validate_bags counts such indices. */
enum { EL_FLAG_HASH_INDICES = 1u };

/* All F embedding tables in one "joint" buffer (--embedding_type joint, same page):
 * table t occupies rows [row_offset[t], row_offset[t+1]) of a row-major
 * [total_rows][dim] array of `dtype`. */
typedef struct {
  void* base;                /* [total_rows][dim], 16-byte aligned; dim * sizeof(dtype) % 16 == 0 */
  const int64_t* row_offset; /* [F+1] device; row_offset[0] = 0, non-decreasing */
  int64_t total_rows;        /* [host] == row_offset[F]; < 2^32 */
  int32_t num_tables;        /* F >= 1 */
  int32_t dim;               /* D >= 1 */
  el_dtype dtype;
  int64_t max_rows;          /* [host] rows of the largest table (>= every
                                row_offset[t+1] - row_offset[t], <= total_rows), or 0 if not
                                known.  Only the embedding-gradient sort reads it: it sorts
                                each table's lookups by their local row, on the fewest bits
                                that hold max_rows - 1 (total_rows - 1 when 0); a value below
                                the largest table's rows breaks that sort (el_validate_bags
                                detects it). */
} el_tables;

/* Lookups in CSR form over F*B bags, table-major: bag (t, b) has number g = t*B + b and
 * holds indices[offsets[g] .. offsets[g+1]) (row numbers local to table t).  A bag may be
 * empty and may repeat a row. */
typedef struct {
  const int32_t* indices; /* [nnz], 4-byte aligned */
  const int32_t* offsets; /* [F*B+1], offsets[0] = 0, non-decreasing, offsets[F*B] = nnz */
  int32_t batch;          /* B >= 0 */
  int64_t nnz;            /* [host] == offsets[F*B]; < 2^31 */
} el_bags;

/*
 * Embedding bag with sum pooling (same page, §Model architecture: one table per
 * categorical feature; the pooling over a CSR bag is the multi-hot generalisation):
 *   emb_out[b][t][:] = sum_{k in bag (t,b), ascending} W_t[indices[k]][:]
 * accumulated in fp32 and rounded once to out_dtype.  An empty bag gives +0.
 * emb_out: [B][F][D] of out_dtype, 16-byte aligned.
 * flags: 0 or EL_FLAG_HASH_INDICES.
 */
EL_API el_status emb_bag_fwd(const el_tables* tab, const el_bags* bags, uint32_t flags, void* emb_out,
                      el_dtype out_dtype, hipStream_t stream);

/*
 * Dot interaction forward (same page, §Model architecture; --interaction_op dot).  With
 * V = F+1 vectors per sample (vector 0 = x0[b], vector 1+t = emb[b][t]) and
 * P = V(V-1)/2 pairs:
 *   out[b][0:D)        = x0[b]                                  (copy)
 *   out[b][D + p(i,j)] = <V_i, V_j>, i > j, p(i,j) = i(i-1)/2 + j (row-major strict lower)
 *   out[b][D+P : out_stride) = +0
 * x0: [B][D], emb: [B][F][D] of in_dtype; out: [B][out_stride] of out_dtype,
 * out_stride >= D + P.  bf16/fp16 inputs use MFMA with fp32 accumulation; fp32 inputs
 * use fp32 FMA.  All base pointers 16-byte aligned.
 */
EL_API el_status dot_interact_fwd(const void* x0, const void* emb, el_dtype in_dtype, int32_t B,
                           int32_t F, int32_t D, void* out, el_dtype out_dtype,
                           int32_t out_stride, hipStream_t stream);

/*
 * The two forward calls in one (same page, §Model architecture: the pooled embeddings and
 * the bottom-MLP output feed the dot interaction).  Same results, bit for bit, as
 *   emb_bag_fwd(tab, bags, flags, emb_out, act_dtype);
 *   dot_interact_fwd(x0, emb_out, act_dtype, B, F, D, out, act_dtype, out_stride);
 * with B = bags->batch, F = tab->num_tables, D = tab->dim.  With emb_out ([B][F][D] of
 * act_dtype, 16-byte aligned) the two kernels run on chunks of samples sized so that each
 * chunk's pooled vectors are read back from the memory-side cache.  emb_out may be NULL
 * when the pooled vectors are not needed (inference): one fused kernel then builds each
 * sample's vectors in on-chip memory and never stores them; it covers bf16 / fp16
 * activations with D % 16 == 0, F <= 64 and out_stride * 2 % 16 == 0 (other shapes:
 * EL_ERR_UNSUPPORTED).  x0: [B][D], out: [B][out_stride] of act_dtype.
 */
EL_API el_status emb_dot_fwd(const el_tables* tab, const el_bags* bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, void* emb_out, void* out,
                             int32_t out_stride, hipStream_t stream);

/*
 * Dot interaction backward.  With G = dout[b] and the symmetric V x V matrix S,
 * S_ij = S_ji = G[D + p(i,j)] (i > j), S_ii = 0:
 *   dV = S V;   dx0[b] = G[0:D) + dV_0;   demb[b][t] = dV_{1+t}
 * Columns [D+P, out_stride) of dout are ignored.  dout: [B][out_stride] of dout_dtype;
 * dx0: [B][D], demb: [B][F][D] of grad_dtype.  fp32 accumulation, one rounding.
 */
EL_API el_status dot_interact_bwd(const void* x0, const void* emb, el_dtype in_dtype, int32_t B,
                           int32_t F, int32_t D, const void* dout, el_dtype dout_dtype,
                           int32_t out_stride, void* dx0, void* demb, el_dtype grad_dtype,
                           hipStream_t stream);

/*
 * The interaction backward with the pooled vectors rebuilt from the tables (same page,
 * §Model architecture: the pooled embeddings are an input of the interaction, so its
 * backward needs them; recomputing them from the tables replaces storing them in the
 * forward and reading them back).  Same results, bit for bit, as
 *   emb_bag_fwd(tab, bags, flags, emb, act_dtype);
 *   dot_interact_bwd(x0, emb, act_dtype, B, F, D, dout, act_dtype, out_stride, dx0, demb,
 *                    grad_dtype);
 * with B = bags->batch, F = tab->num_tables, D = tab->dim; the pooled vectors are never
 * stored.  The tables must not change between the forward and this call.  x0: [B][D] and
 * dout: [B][out_stride] of act_dtype (bf16 or fp16); dx0: [B][D], demb: [B][F][D] of
 * grad_dtype; all 16-byte aligned.  One fused kernel; it covers D % 16 == 0, D >= 32,
 * F <= 31, (F+1)/2 * D/8 <= 256 (one row pair and column block per thread) and
 * out_stride % 8 == 0 (other shapes, fp32 activations: EL_ERR_UNSUPPORTED, nothing
 * enqueued).  Bags of any length are correct; one-lookup bags take the pipelined path.
 */
EL_API el_status emb_dot_bwd(const el_tables* tab, const el_bags* bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, const void* dout,
                             int32_t out_stride, void* dx0, void* demb, el_dtype grad_dtype,
                             hipStream_t stream);

/*
 * The "cat" interaction (same page, §Command-line options, --interaction_op cat): the
 * sample's V = F+1 vectors side by side instead of their pairwise dot products,
 *   out[b] = [ x0[b] | emb[b][0] | ... | emb[b][F-1] | +0 pad ]   (V*D values, then zeros)
 * The bottom-MLP output the model concatenates with the interaction output is the first
 * block itself (it appears once).  x0: [B][D], emb: [B][F][D] of in_dtype; out:
 * [B][out_stride] of out_dtype, out_stride >= (F+1)*D; one rounding per value (equal dtypes
 * copy bits).  All base pointers 16-byte aligned.
 */
EL_API el_status cat_interact_fwd(const void* x0, const void* emb, el_dtype in_dtype, int32_t B,
                                  int32_t F, int32_t D, void* out, el_dtype out_dtype,
                                  int32_t out_stride, hipStream_t stream);

/*
 * Backward of the cat interaction: every vector's gradient is its own block of the upstream
 * gradient G = dout[b]:  dx0[b] = G[0:D),  demb[b][t] = G[D(1+t) : D(2+t)).  Columns
 * [(F+1)*D, out_stride) of dout are ignored.  dout: [B][out_stride] of dout_dtype; dx0:
 * [B][D], demb: [B][F][D] of grad_dtype; 16-byte aligned.
 */
EL_API el_status cat_interact_bwd(const void* dout, el_dtype dout_dtype, int32_t B, int32_t F,
                                  int32_t D, int32_t out_stride, void* dx0, void* demb,
                                  el_dtype grad_dtype, hipStream_t stream);

/*
 * emb_bag_fwd and cat_interact_fwd in one call: the same bits as
 *   emb_bag_fwd(tab, bags, flags, emb, act_dtype);
 *   cat_interact_fwd(x0, emb, act_dtype, B, F, D, out, act_dtype, out_stride);
 * with B = bags->batch, F = tab->num_tables, D = tab->dim, but each pooled vector is written
 * straight into its block of the output row (the pooled vectors are not stored anywhere
 * else).  x0: [B][D], out: [B][out_stride] of act_dtype, out_stride >= (F+1)*D;
 * D * sizeof(act_dtype) and out_stride * sizeof(act_dtype) multiples of 16 bytes (else
 * EL_ERR_UNSUPPORTED, nothing enqueued); 16-byte aligned.
 */
EL_API el_status emb_cat_fwd(const el_tables* tab, const el_bags* bags, uint32_t flags,
                             const void* x0, el_dtype act_dtype, void* out, int32_t out_stride,
                             hipStream_t stream);

/* [host, pure] Bytes of device workspace that emb_grad_reduce_update and emb_grad_sort
 * need for these tables and bags (0 when nnz == 0).  Returns 0 for invalid arguments. */
EL_API size_t emb_grad_workspace_bytes(const el_tables* tab, const el_bags* bags);

/*
 * Sparse SGD update of the embedding rows (same page, §Command-line options, --lr: plain
 * SGD).  For every distinct row r looked up by the batch:
 *   W[r] <- round( W[r] - lr * sum_{lookups k of row r, in lookup order} demb[b_k][t_k] )
 * Rows that are not looked up are not written.  The lookups are sorted by joint row with a
 * stable, deterministic LSD radix sort (each table's lookups by local row, on the bits of
 * tab->max_rows); equal rows form runs that are summed in sorted order (fp32) in ranges of
 * consecutive lookups, with an ordered fix-up for runs spanning ranges.  No floating-point
 * atomics (the sort's digit histograms count with integer LDS atomics, exact in any order):
 * the result is bitwise reproducible, whatever the launch configuration.
 * demb: [B][F][D] of grad_dtype, 16-byte aligned.  workspace: >= emb_grad_workspace_bytes,
 * 256-byte aligned, contents on entry irrelevant.
 */
EL_API el_status emb_grad_reduce_update(const el_tables* tab, const el_bags* bags, uint32_t flags,
                                 const void* demb, el_dtype grad_dtype, float lr,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * emb_grad_reduce_update for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * computation, bit for bit, with the workspace taken from a static scratch array that the
 * library holds on every GPU it runs on (EL_NOALLOC_SCRATCH_BYTES per GPU, kept until the
 * process ends) instead of a caller-provided buffer.  The caller still passes the tables,
 * the bags and demb as for emb_grad_reduce_update.  A call whose workspace would exceed
 * the scratch (emb_grad_workspace_bytes(tab, bags) > EL_NOALLOC_SCRATCH_BYTES) returns
 * EL_ERR_WORKSPACE and enqueues nothing.  The call allocates nothing: no hipMalloc or
 * hipFree, no allocating library routine.  Nothing in the scratch needs clearing: every
 * byte a call reads it has written first.  All calls on one GPU share that GPU's scratch, so
 * two calls that may overlap on one GPU (other streams, other threads) race; the caller
 * orders them.
 */
#define EL_NOALLOC_SCRATCH_BYTES (64u << 20)
EL_API el_status emb_grad_reduce_update_noalloc(const el_tables* tab, const el_bags* bags,
                                                uint32_t flags, const void* demb,
                                                el_dtype grad_dtype, float lr, hipStream_t stream);

/*
 * emb_grad_reduce_update in two halves, so that the sort -- which depends only on the
 * lookups -- can run on another stream while the forward and the interaction backward
 * produce demb:
 *   emb_grad_prepare: builds the (row, bag) keys of every lookup and sorts them into the
 *     workspace;
 *   emb_grad_apply:   the segment reduce of demb and the SGD row update, from the sorted
 *     lookups that emb_grad_prepare left in the same workspace.
 * prepare followed by apply gives bitwise the result of emb_grad_reduce_update.  Both calls
 * take the same tables, bags and flags; the caller orders them (same stream, or an event
 * between streams) and leaves the workspace and the index / offset arrays untouched in
 * between.  Arguments as for emb_grad_reduce_update.
 */
EL_API el_status emb_grad_prepare(const el_tables* tab, const el_bags* bags, uint32_t flags,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);
EL_API el_status emb_grad_apply(const el_tables* tab, const el_bags* bags, uint32_t flags,
                                const void* demb, el_dtype grad_dtype, float lr,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The sort and segment stage of emb_grad_reduce_update, exposed for inspection:
 *   sorted_rows[q], bag_ids[q] (q < nnz): global row (row_offset[t] + index) and bag id
 *     g = t*B + b of every lookup, sorted by row, equal rows in lookup order;
 *   unique_rows[u] (u < U): the distinct rows ascending; seg_offsets[u]: first sorted
 *     position of unique row u, seg_offsets[U] = nnz; num_unique[0] = U.
 * Arrays: sorted_rows, bag_ids, unique_rows [nnz]; seg_offsets [nnz+1]; num_unique [1].
 */
EL_API el_status emb_grad_sort(const el_tables* tab, const el_bags* bags, uint32_t flags,
                        void* workspace, size_t workspace_bytes, uint32_t* sorted_rows,
                        uint32_t* bag_ids, uint32_t* unique_rows, uint32_t* seg_offsets,
                        uint32_t* num_unique, hipStream_t stream);

/*
 * Count defects of a CSR batch: offsets that decrease, offsets[0] != 0,
 * offsets[F*B] != nnz, (without EL_FLAG_HASH_INDICES) indices outside their table, and
 * (when tab->max_rows > 0) tables with more than max_rows rows.
 * bad_count: [1] int64 device, overwritten with the total.  A grid of workgroups scans the
 * bags; their subtotals are added with integer atomics (the count is exact whatever the
 * order).  Not part of the computation.
 */
EL_API el_status el_validate_bags(const el_tables* tab, const el_bags* bags, uint32_t flags,
                           int64_t* bad_count, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Dense layers, logistic loss and dense SGD: the steps on either side of the core (same
 * page, §Model architecture: the bottom MLP is a series of linear layers with ReLU
 * activations; the top MLP is a series of dense layers ending in one number, the click
 * likelihood; §Command-line options: --bottom_mlp_sizes 512,256,128 and --top_mlp_sizes
 * 1024,1024,512,256,1; the MLPs train in mixed precision with fp32 master weights).
 * Activations and weights are 16-bit (EL_BF16 or EL_F16, one dtype per call) and every
 * product accumulates in fp32 (MFMA); weight / bias gradients are fp32.  Weights are
 * w[n][k], row-major [N][K]: input feature k -> output feature n.
 * ------------------------------------------------------------------------------------ */
enum { EL_ACT_NONE = 0u, EL_ACT_RELU = 1u };
enum { EL_LINEAR_DX_RELU_MASK = 1u };

/*
 * Dense layer forward:  y[m][n] = act( sum_k x[m][k] * w[n][k] + bias[n] ),  m < M, n < N.
 * x: [M] rows of stride ldx (first K used); w: [N][K]; bias: fp32 [N] or NULL; y: [M] rows
 * of stride ldy (first N written), one rounding per output.  act: EL_ACT_NONE or
 * EL_ACT_RELU.  Shapes: K % 8 == 0, ldx % 8 == 0, N == 1 or N % 8 == 0 (then ldy % 8 == 0);
 * N == 1 takes K <= 2048 (other shapes EL_ERR_UNSUPPORTED).  x, w, bias 16-byte aligned;
 * y 16-byte aligned (2-byte when N == 1).  A K not divisible by 8 is served by zero-padding
 * the inputs and the weight columns, which leaves every output unchanged.
 */
EL_API el_status el_linear_fwd(const void* x, int32_t ldx, int32_t M, int32_t K, const void* w,
                               const float* bias, int32_t N, uint32_t act, void* y, int32_t ldy,
                               el_dtype dtype, hipStream_t stream);

/* [host, pure] Bytes of device workspace el_linear_bwd needs for these sizes (a transposed
 * copy of w for the data gradient, and the fp32 partial sums of the weight gradient's
 * batch slices); 0 for invalid sizes or M == 0. */
EL_API size_t el_linear_bwd_workspace_bytes(int32_t M, int32_t K, int32_t N);

/*
 * Dense layer backward, from dz = dL/d(pre-activation) [M] rows of stride ldz:
 *   dx[m][k] = sum_n dz[m][n] w[n][k]      (dx may be NULL: not computed)
 *              times 1[x[m][k] > 0] with EL_LINEAR_DX_RELU_MASK (x is then the output of a
 *              ReLU layer below, and dx is that layer's dz)
 *   dw[n][k] = sum_m dz[m][n] x[m][k]      fp32 [N][K], overwritten
 *   db[n]    = sum_m dz[m][n]              fp32 [N], overwritten
 * The sums over m are split into fixed slices whose fp32 partials are added in slice order:
 * bitwise reproducible.  dx: [M] rows of stride lddx (lddx % 8 == 0, 16-byte aligned); x,
 * w, dz as for el_linear_fwd (dz has the shape of y).  workspace: >=
 * el_linear_bwd_workspace_bytes(M, K, N), 256-byte aligned (may be NULL when that is 0).
 */
EL_API el_status el_linear_bwd(const void* x, int32_t ldx, int32_t M, int32_t K, const void* w,
                               int32_t N, const void* dz, int32_t ldz, void* dx, int32_t lddx,
                               uint32_t flags, float* dw, float* db, el_dtype dtype,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of a ReLU from its output y:  dz[m][n] = dy[m][n] * 1[y[m][n] > 0]  (the bottom
 * MLP's last ReLU, between the interaction gradient dx0 and the last bottom layer).
 * dy, y, dz: [M] rows of stride ld, first N used; N % 8 == 0, ld % 8 == 0; 16-byte aligned.
 */
EL_API el_status el_relu_bwd(const void* dy, const void* y, void* dz, int32_t M, int32_t N,
                             int32_t ld, el_dtype dtype, hipStream_t stream);

/* [host, pure] Bytes of device workspace el_bce_logits needs for M samples (per-workgroup
 * partial sums of the loss); 0 for M < 1. */
EL_API size_t el_bce_workspace_bytes(int32_t M);

/*
 * Logistic loss of one logit per sample (the model's output read as a click likelihood;
 * the page names no loss, binary cross-entropy is the plain reading), batch mean:
 *   loss[0] = (1/M) sum_m [ max(z_m, 0) - z_m y_m + log(1 + exp(-|z_m|)) ]   (fp32)
 *   dz[m]   = (sigmoid(z_m) - y_m) / M                                       (dtype)
 * z: logits at z[m * ldz]; labels: fp32 [M] in {0, 1}; dz at dz[m * lddz].  The loss terms
 * are summed in double in a fixed order (per-workgroup partials in workspace, then in
 * workgroup order): bitwise reproducible.  workspace: >= el_bce_workspace_bytes(M),
 * 8-byte aligned.
 */
EL_API el_status el_bce_logits(const void* z, int32_t ldz, const float* labels, int32_t M,
                               el_dtype dtype, float* loss, void* dz, int32_t lddz,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Plain SGD on dense parameters kept in fp32 (--lr, same page):
 *   master[i] <- master[i] - lr * grad[i]   (one fp32 rounding),   copy[i] <- master[i]
 * rounded to copy_dtype (EL_BF16 / EL_F16; copy may be NULL).  n elements.
 */
EL_API el_status el_sgd_dense(float* master, void* copy, el_dtype copy_dtype, const float* grad,
                              int64_t n, float lr, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Measurement helper: HBM calibration.  The page measures throughput (samples/s, warm-up
 * excluded, §Training performance benchmark); since every kernel of this library is
 * bandwidth-bound, the bandwidth that plain streaming kernels reach on the same GPU is the
 * yardstick its kernels are compared with (beside the published peak).  One call runs one
 * kernel (k_copy_calib / k_gather_calib) that moves 16-byte vectors, 8 loads in flight per
 * thread, over the whole buffer (streams in workgroup chunks of 32 KiB).  `bytes` is the
 * total traffic (reads + writes):
 *   EL_CALIB_READ          reads src[0, bytes); writes 8 MiB of per-thread xors to dst;
 *   EL_CALIB_WRITE         writes dst[0, bytes);
 *   EL_CALIB_COPY          copies src[0, bytes/2) to dst[0, bytes/2);
 *   EL_CALIB_READ3_WRITE1  reads src[0, 3*bytes/4) and writes dst[0, bytes/4), output
 *                          vector i the xor of input vectors i, i + m and i + 2m (m = bytes/64
 *                          output vectors: three read streams and one write stream);
 *   EL_CALIB_GATHER        reads the nrows rows idx[i] (row_bytes each, 16..1024, a multiple
 *                          of 16) of the row-major table at src and writes the first `bytes`
 *                          of each (0: the whole row) to dst[i * bytes] (traffic = nrows *
 *                          (row_bytes + bytes) plus the indices);
 *   EL_CALIB_GATHER_READ   the same rows, only read (8 MiB of per-thread xors to dst).
 * OR-ing EL_CALIB_NT_LOADS / EL_CALIB_NT_STORES into the mode makes the kernel's data loads /
 * stores non-temporal (the cache policy that is faster depends on the mix).
 * Pointers 16-byte aligned; bytes a multiple of 64.  Not part of the model's computation.
 * ------------------------------------------------------------------------------------ */
enum { EL_CALIB_READ = 0, EL_CALIB_WRITE = 1, EL_CALIB_COPY = 2, EL_CALIB_READ3_WRITE1 = 3,
       EL_CALIB_GATHER = 4, EL_CALIB_GATHER_READ = 5,
       EL_CALIB_MODE_MASK = 15, EL_CALIB_NT_LOADS = 16, EL_CALIB_NT_STORES = 32 };
EL_API el_status el_hbm_calib(int32_t mode, const void* src, void* dst, size_t bytes,
                              const int32_t* idx, int64_t nrows, int32_t row_bytes,
                              hipStream_t stream);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
EL_API const char* el_last_error(void);

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
EL_API int el_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EMBCORE_H */
