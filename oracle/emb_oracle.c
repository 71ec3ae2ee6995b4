/*
 * emb_oracle.c -- plain, slow, single-threaded CPU oracle for the sparse-embedding +
 * dot-interaction core of a DLRM-style recommender.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or helper
 * with the HIP library: it has its own dtype codes and its own number converters.
 *
 * What it follows (page "DLRM For PyTorch"):
 *   - §Model architecture: one embedding table per categorical feature; the bottom-MLP
 *     output and the embedding vectors go into a "dot interaction"; its output is
 *     concatenated with the bottom-MLP output.  The pairwise products are taken over the
 *     strict lower triangle of the (F+1) x (F+1) Gram matrix of the vectors of a sample.
 *   - §Command-line options, --hash_indices: an index is replaced by index mod table size.
 *   - §Command-line options, --lr / --embedding_dim: plain SGD on the embedding rows.
 *   - §Model architecture and --bottom_mlp_sizes / --top_mlp_sizes: the dense layers of the
 *     bottom and top MLPs (forward, backward), a logistic loss on the final logit, and plain
 *     SGD on the dense parameters.
 * Where the page is silent (sum pooling over CSR bags, pair order, concat order, zero
 * padding, rounding), the plainest reading is taken; the readings are listed in the
 * repository's design notes.
 *
 * Arithmetic: every stored input value is widened exactly to double; all sums are in
 * double, in a fixed ascending loop order; every output is rounded ONCE to its output
 * format with round-to-nearest-even (no flush to zero, overflow to +-inf, NaN stays NaN).
 *
 * Error behaviour: functions return 0 on success, a negative code on bad input (an index
 * outside its table, non-monotone offsets, unknown dtype, allocation failure).
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes of the oracle (independent of any other component) */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F64 = 3 };

enum {
  OR_OK = 0,
  OR_BAD_DTYPE = -1,
  OR_BAD_INDEX = -2,
  OR_BAD_OFFSETS = -3,
  OR_NO_MEMORY = -4,
  OR_BAD_SHAPE = -5
};

/* ------------------------------------------------------------------------------------ */
/* Number formats                                                                        */
/* ------------------------------------------------------------------------------------ */

/* Exact widening of a bfloat16 bit pattern: bf16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Exact widening of an IEEE binary16 bit pattern (1 sign, 5 exponent, 10 fraction bits). */
static double f16_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24); /* subnormal: frac * 2^-24 */
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
  }
  return sign ? -v : v;
}

/*
 * Round a double to the nearest value of a binary format with `p` significand bits
 * (hidden bit included) and minimum normal exponent `emin`, ties to even.  Returns the
 * rounded value as a double (exact), or +-inf when it exceeds `maxfinite`.
 * This is the textbook definition: the quantum at the value's binade is 2^(E-p+1) with
 * E = max(floor(log2|x|), emin); the value is divided by the quantum (exact, a power of
 * two), rounded to an integer with ties to even, and scaled back.
 */
static double round_to_format(double x, int p, int emin, double maxfinite) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  double a = fabs(x);
  int e2;
  frexp(a, &e2);  /* a = m * 2^e2, m in [0.5, 1) */
  int E = e2 - 1; /* a in [2^E, 2^(E+1)) */
  if (E < emin) E = emin;
  double quantum = ldexp(1.0, E - (p - 1));
  double n = a / quantum;          /* exact */
  double r = nearbyint(n) * quantum; /* nearbyint: current mode, round-to-nearest-even */
  if (r > maxfinite) r = INFINITY;
  return x < 0 ? -r : r;
}

static uint16_t double_to_bf16_bits(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xffc0 : 0x7fc0);
  /* bfloat16: 8 significand bits, emin -126, max (2 - 2^-7) * 2^127 */
  double r = round_to_format(x, 8, -126, ldexp(255.0, 120));
  float f = (float)r; /* exact: every bf16 value is a binary32 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static uint16_t double_to_f16_bits(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xfe00 : 0x7e00);
  /* binary16: 11 significand bits, emin -14, max 65504 */
  double r = round_to_format(x, 11, -14, 65504.0);
  uint16_t sign = signbit(r) ? 0x8000 : 0;
  double a = fabs(r);
  if (isinf(a)) return sign | 0x7c00;
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -14)) { /* subnormal: a = frac * 2^-24 */
    return sign | (uint16_t)(a / ldexp(1.0, -24));
  }
  int e2;
  frexp(a, &e2);
  int E = e2 - 1;
  uint16_t frac = (uint16_t)(a / ldexp(1.0, E - 10) - 1024.0);
  return sign | (uint16_t)((E + 15) << 10) | frac;
}

static double load_elem(const void* base, int dtype, size_t i) {
  switch (dtype) {
    case OR_F32: return (double)((const float*)base)[i];
    case OR_F16: return f16_bits_to_double(((const uint16_t*)base)[i]);
    case OR_BF16: return bf16_bits_to_double(((const uint16_t*)base)[i]);
    case OR_F64: return ((const double*)base)[i];
  }
  return NAN;
}

static void store_elem(void* base, int dtype, size_t i, double v) {
  switch (dtype) {
    case OR_F32: ((float*)base)[i] = (float)v; break; /* C conversion: round to nearest even */
    case OR_F16: ((uint16_t*)base)[i] = double_to_f16_bits(v); break;
    case OR_BF16: ((uint16_t*)base)[i] = double_to_bf16_bits(v); break;
    case OR_F64: ((double*)base)[i] = v; break;
  }
}

static int dtype_ok(int d) { return d == OR_F32 || d == OR_F16 || d == OR_BF16 || d == OR_F64; }

/* Batch converters, exported so that the test suite can pin them against other libraries. */
void oracle_round_f64(const double* x, int64_t n, int dtype, void* out) {
  for (int64_t i = 0; i < n; ++i) store_elem(out, dtype, (size_t)i, x[i]);
}
void oracle_widen(const void* x, int64_t n, int dtype, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = load_elem(x, dtype, (size_t)i);
}

/* ------------------------------------------------------------------------------------ */
/* Index handling                                                                        */
/* ------------------------------------------------------------------------------------ */

/* --hash_indices: index := index mod table size; the remainder is taken with the sign of
 * the divisor (floor modulo), so that a negative index also lands inside the table. */
static int64_t floor_mod(int64_t a, int64_t n) {
  int64_t r = a % n;
  return r < 0 ? r + n : r;
}

/* Resolve lookup k of table t to a global row of the joint table, or -1 if out of range. */
static int64_t resolve_row(const int64_t* row_offset, int t, int32_t idx, int hash) {
  int64_t n = row_offset[t + 1] - row_offset[t];
  int64_t r = idx;
  if (hash) r = floor_mod(r, n);
  if (r < 0 || r >= n) return -1;
  return row_offset[t] + r;
}

static int check_offsets(const int32_t* offsets, int64_t nbags) {
  if (offsets[0] != 0) return OR_BAD_OFFSETS;
  for (int64_t g = 0; g < nbags; ++g)
    if (offsets[g + 1] < offsets[g]) return OR_BAD_OFFSETS;
  return OR_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Forward: embedding bag with sum pooling                                               */
/* ------------------------------------------------------------------------------------ */

/*
 * emb[b][t][:] = sum over the lookups k of bag (t, b), in ascending k, of the table row
 * W_t[idx[k]].  Bags are table-major: bag (t, b) is number g = t*B + b and holds the
 * lookups offsets[g] .. offsets[g+1]-1.  The joint table stores table t at rows
 * row_offset[t] .. row_offset[t+1]-1 of a [total_rows][D] array.
 * The sum of a non-empty bag is x_1 + x_2 + ... + x_n, starting from its first row, so a
 * one-row bag returns that row exactly (sign of zero included: the hotness-1 gather is an
 * index select).  An empty bag gives +0.
 */
int oracle_emb_bag_fwd(const void* W, int w_dtype, const int64_t* row_offset, int F, int D,
                       const int32_t* indices, const int32_t* offsets, int B, int hash,
                       void* out, int out_dtype) {
  if (!dtype_ok(w_dtype) || !dtype_ok(out_dtype)) return OR_BAD_DTYPE;
  if (F < 1 || D < 1 || B < 0) return OR_BAD_SHAPE;
  int64_t nbags = (int64_t)F * B;
  int rc = check_offsets(offsets, nbags);
  if (rc) return rc;
  int bad = 0, nomem = 0;
  /* Bags are independent; an OpenMP build splits them over threads (same arithmetic per
   * bag, so the same bits); the plain build ignores the pragmas. */
#pragma omp parallel reduction(| : bad, nomem)
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!acc) nomem = 1;
#pragma omp for collapse(2) schedule(static)
    for (int t = 0; t < F; ++t) {
      for (int b = 0; b < B; ++b) {
        if (!acc) continue;
        int64_t g = (int64_t)t * B + b;
        for (int d = 0; d < D; ++d) acc[d] = 0.0;
        for (int64_t k = offsets[g]; k < offsets[g + 1]; ++k) {
          int64_t row = resolve_row(row_offset, t, indices[k], hash);
          if (row < 0) { bad = 1; break; }
          for (int d = 0; d < D; ++d) {
            double w = load_elem(W, w_dtype, (size_t)row * D + d);
            acc[d] = (k == offsets[g]) ? w : acc[d] + w;
          }
        }
        for (int d = 0; d < D; ++d)
          store_elem(out, out_dtype, ((size_t)b * F + t) * D + d, acc[d]);
      }
    }
    free(acc);
  }
  if (nomem) return OR_NO_MEMORY;
  if (bad) return OR_BAD_INDEX;
  return OR_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Dot interaction                                                                       */
/* ------------------------------------------------------------------------------------ */

/* Position of pair (i, j), i > j, in the row-major strict lower triangle:
 * (1,0), (2,0), (2,1), (3,0), ...  */
static int64_t pair_index(int i, int j) { return (int64_t)i * (i - 1) / 2 + j; }

/* Vector v of sample b: vector 0 is the bottom-MLP output x0[b], vector 1+t is the
 * pooled embedding of table t. */
static double vec_elem(const void* x0, const void* emb, int dtype, int b, int F, int D, int v,
                       int d) {
  if (v == 0) return load_elem(x0, dtype, (size_t)b * D + d);
  return load_elem(emb, dtype, ((size_t)b * F + (v - 1)) * D + d);
}

/*
 * out[b] = [ x0[b] (D values) | <V_i, V_j> for i > j in row-major order (P values) | +0 pad ]
 * with V = F + 1 vectors per sample, P = V(V-1)/2, and out_stride >= D + P.
 */
int oracle_dot_interact_fwd(const void* x0, const void* emb, int in_dtype, int B, int F, int D,
                            void* out, int out_dtype, int out_stride) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return OR_BAD_DTYPE;
  int V = F + 1;
  int64_t P = (int64_t)V * (V - 1) / 2;
  if (F < 1 || D < 1 || B < 0 || out_stride < D + P) return OR_BAD_SHAPE;
#pragma omp parallel for schedule(static)
  for (int b = 0; b < B; ++b) {
    size_t row = (size_t)b * out_stride;
    for (int d = 0; d < D; ++d) store_elem(out, out_dtype, row + d, vec_elem(x0, emb, in_dtype, b, F, D, 0, d));
    for (int i = 1; i < V; ++i) {
      for (int j = 0; j < i; ++j) {
        double s = 0.0;
        for (int d = 0; d < D; ++d)
          s += vec_elem(x0, emb, in_dtype, b, F, D, i, d) * vec_elem(x0, emb, in_dtype, b, F, D, j, d);
        store_elem(out, out_dtype, row + D + pair_index(i, j), s);
      }
    }
    for (int64_t c = D + P; c < out_stride; ++c) store_elem(out, out_dtype, row + c, 0.0);
  }
  return OR_OK;
}

/*
 * Backward of the interaction for an upstream gradient G = dout[b] (padding ignored).
 * The pair outputs depend on the vectors through Z_ij = <V_i, V_j>; with the symmetric
 * matrix S (S_ij = S_ji = G[D + p(i,j)] for i > j, zero diagonal), the gradient of
 * sum_p G_p Z_p with respect to V_k is dV_k = sum_j S_kj V_j.  The first D outputs are a
 * copy of x0, so dx0 = G[0:D) + dV_0 and demb[b][t] = dV_{1+t}.
 */
int oracle_dot_interact_bwd(const void* x0, const void* emb, int in_dtype, int B, int F, int D,
                            const void* dout, int dout_dtype, int out_stride, void* dx0,
                            void* demb, int grad_dtype) {
  if (!dtype_ok(in_dtype) || !dtype_ok(dout_dtype) || !dtype_ok(grad_dtype)) return OR_BAD_DTYPE;
  int V = F + 1;
  int64_t P = (int64_t)V * (V - 1) / 2;
  if (F < 1 || D < 1 || B < 0 || out_stride < D + P) return OR_BAD_SHAPE;
#pragma omp parallel for schedule(static)
  for (int b = 0; b < B; ++b) {
    size_t row = (size_t)b * out_stride;
    for (int k = 0; k < V; ++k) {
      for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int j = 0; j < V; ++j) {
          if (j == k) continue; /* zero diagonal */
          int hi = k > j ? k : j, lo = k > j ? j : k;
          double s = load_elem(dout, dout_dtype, row + D + pair_index(hi, lo));
          acc += s * vec_elem(x0, emb, in_dtype, b, F, D, j, d);
        }
        if (k == 0)
          store_elem(dx0, grad_dtype, (size_t)b * D + d, load_elem(dout, dout_dtype, row + d) + acc);
        else
          store_elem(demb, grad_dtype, ((size_t)b * F + (k - 1)) * D + d, acc);
      }
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------------------ */
/* "cat" interaction (--interaction_op cat)                                              */
/* ------------------------------------------------------------------------------------ */

/*
 * The interaction that concatenates instead of multiplying: out[b] = [ V_0 | V_1 | ... |
 * V_F | +0 pad ], the sample's V = F + 1 vectors (V_0 = x0[b], V_{1+t} = the pooled
 * embedding of table t), D values each, one after another, then zeros up to out_stride
 * >= V*D.  The bottom-MLP output the model concatenates with the interaction output is
 * V_0 itself, so it appears once.  Each value is rounded once to out_dtype.
 */
int oracle_cat_interact_fwd(const void* x0, const void* emb, int in_dtype, int B, int F, int D,
                            void* out, int out_dtype, int out_stride) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return OR_BAD_DTYPE;
  int V = F + 1;
  if (F < 1 || D < 1 || B < 0 || out_stride < (int64_t)V * D) return OR_BAD_SHAPE;
  for (int b = 0; b < B; ++b) {
    size_t row = (size_t)b * out_stride;
    for (int v = 0; v < V; ++v)
      for (int d = 0; d < D; ++d)
        store_elem(out, out_dtype, row + (size_t)v * D + d, vec_elem(x0, emb, in_dtype, b, F, D, v, d));
    for (int64_t c = (int64_t)V * D; c < out_stride; ++c) store_elem(out, out_dtype, row + c, 0.0);
  }
  return OR_OK;
}

/*
 * Backward of the cat interaction for an upstream gradient G = dout[b]: each output value
 * is one element of one vector, so a vector's gradient is its own block of G:
 * dx0[b] = G[0:D), demb[b][t] = G[D(1+t) : D(2+t)).  Padding columns are ignored.
 */
int oracle_cat_interact_bwd(const void* dout, int dout_dtype, int B, int F, int D, int out_stride,
                            void* dx0, void* demb, int grad_dtype) {
  if (!dtype_ok(dout_dtype) || !dtype_ok(grad_dtype)) return OR_BAD_DTYPE;
  int V = F + 1;
  if (F < 1 || D < 1 || B < 0 || out_stride < (int64_t)V * D) return OR_BAD_SHAPE;
  for (int b = 0; b < B; ++b) {
    size_t row = (size_t)b * out_stride;
    for (int d = 0; d < D; ++d)
      store_elem(dx0, grad_dtype, (size_t)b * D + d, load_elem(dout, dout_dtype, row + d));
    for (int t = 0; t < F; ++t)
      for (int d = 0; d < D; ++d)
        store_elem(demb, grad_dtype, ((size_t)b * F + t) * D + d,
                   load_elem(dout, dout_dtype, row + (size_t)(1 + t) * D + d));
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Embedding-gradient sort, run-length segments, reduce + SGD row update                 */
/* ------------------------------------------------------------------------------------ */

typedef struct {
  uint32_t key; /* global row of the joint table */
  uint32_t val; /* bag id g = t*B + b */
  int64_t pos;  /* lookup position k, the tie-break that makes the sort stable */
} kv_t;

static int kv_cmp(const void* a, const void* b) {
  const kv_t* x = (const kv_t*)a;
  const kv_t* y = (const kv_t*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
  return 0;
}

/* Build (row, bag) for every lookup and sort by row, ties in lookup order (= stable). */
static int build_sorted(const int64_t* row_offset, int F, const int32_t* indices,
                        const int32_t* offsets, int B, int hash, kv_t** out_kv, int64_t* out_n) {
  int64_t nbags = (int64_t)F * B;
  int rc = check_offsets(offsets, nbags);
  if (rc) return rc;
  int64_t n = offsets[nbags];
  kv_t* kv = (kv_t*)malloc(sizeof(kv_t) * (size_t)(n > 0 ? n : 1));
  if (!kv) return OR_NO_MEMORY;
  for (int t = 0; t < F; ++t) {
    for (int b = 0; b < B; ++b) {
      int64_t g = (int64_t)t * B + b;
      for (int64_t k = offsets[g]; k < offsets[g + 1]; ++k) {
        int64_t row = resolve_row(row_offset, t, indices[k], hash);
        if (row < 0) { free(kv); return OR_BAD_INDEX; }
        kv[k].key = (uint32_t)row;
        kv[k].val = (uint32_t)g;
        kv[k].pos = k;
      }
    }
  }
  qsort(kv, (size_t)n, sizeof(kv_t), kv_cmp);
  *out_kv = kv;
  *out_n = n;
  return OR_OK;
}

/*
 * sorted_rows[q], bag_ids[q]: the (row, bag) pairs of all lookups, sorted by row, equal
 * rows in lookup order.  unique_rows[u]: the distinct rows ascending; seg_offsets[u]: first
 * sorted position of unique row u, seg_offsets[U] = nnz; *num_unique = U.
 */
int oracle_grad_sort(const int64_t* row_offset, int F, const int32_t* indices,
                     const int32_t* offsets, int B, int hash, uint32_t* sorted_rows,
                     uint32_t* bag_ids, uint32_t* unique_rows, uint32_t* seg_offsets,
                     uint32_t* num_unique) {
  kv_t* kv = NULL;
  int64_t n = 0;
  int rc = build_sorted(row_offset, F, indices, offsets, B, hash, &kv, &n);
  if (rc) return rc;
  uint32_t u = 0;
  for (int64_t q = 0; q < n; ++q) {
    sorted_rows[q] = kv[q].key;
    bag_ids[q] = kv[q].val;
    if (q == 0 || kv[q].key != kv[q - 1].key) {
      unique_rows[u] = kv[q].key;
      seg_offsets[u] = (uint32_t)q;
      ++u;
    }
  }
  seg_offsets[u] = (uint32_t)n;
  *num_unique = u;
  free(kv);
  return OR_OK;
}

/*
 * Sparse SGD: for every distinct row r touched by the batch,
 *   W[r] <- round( W[r] - lr * sum_{lookups k with row r, in sorted order} demb[b_k][t_k] )
 * and every other row is left as it is (its gradient is zero).  lr is the binary32 value
 * the caller passes, widened exactly.  W is updated in place.
 */
int oracle_grad_reduce_update(void* W, int w_dtype, const int64_t* row_offset, int F, int D,
                              const int32_t* indices, const int32_t* offsets, int B, int hash,
                              const void* demb, int grad_dtype, float lr) {
  if (!dtype_ok(w_dtype) || !dtype_ok(grad_dtype)) return OR_BAD_DTYPE;
  if (F < 1 || D < 1 || B < 0) return OR_BAD_SHAPE;
  kv_t* kv = NULL;
  int64_t n = 0;
  int rc = build_sorted(row_offset, F, indices, offsets, B, hash, &kv, &n);
  if (rc) return rc;
  double* acc = (double*)malloc(sizeof(double) * (size_t)D);
  if (!acc) { free(kv); return OR_NO_MEMORY; }
  int64_t q = 0;
  while (q < n) {
    uint32_t row = kv[q].key;
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    for (; q < n && kv[q].key == row; ++q) {
      uint32_t g = kv[q].val;
      int64_t t = g / (uint32_t)B, b = g % (uint32_t)B;
      for (int d = 0; d < D; ++d) acc[d] += load_elem(demb, grad_dtype, ((size_t)b * F + t) * D + d);
    }
    for (int d = 0; d < D; ++d) {
      size_t i = (size_t)row * D + d;
      store_elem(W, w_dtype, i, load_elem(W, w_dtype, i) - (double)lr * acc[d]);
    }
  }
  free(acc);
  free(kv);
  return OR_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Dense layers, logistic loss, dense SGD                                                */
/* ------------------------------------------------------------------------------------ */
/*
 * Page "DLRM For PyTorch", §Model architecture: the dense features go through the bottom
 * MLP, a series of linear layers each followed by a ReLU; the concatenated interaction
 * output goes through the top MLP, a series of dense layers with activations, and the model
 * ends in one number read as the likelihood of a click.  §Command-line options gives the
 * layer widths (--bottom_mlp_sizes 512,256,128; --top_mlp_sizes 1024,1024,512,256,1).
 * The page names no loss; a click likelihood from one logit is read as the logistic
 * (binary cross-entropy) loss, averaged over the batch.  Weights follow the usual dense
 * layer layout: w[n][k] maps input feature k to output feature n.
 */

/*
 * Forward of one dense layer:
 *   y[m][n] = act( sum_k x[m][k] * w[n][k] + bias[n] ),   act = ReLU (max(., 0)) or identity.
 * x is [M] rows of stride ldx (the first K used), w is [N][K], bias is fp32 [N] or NULL,
 * y is [M] rows of stride ldy (the first N written).  One rounding per output.
 */
int oracle_linear_fwd(const void* x, int x_dtype, int M, int K, int ldx, const void* w,
                      int w_dtype, int N, const float* bias, int relu, void* y, int y_dtype,
                      int ldy) {
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype) || !dtype_ok(y_dtype)) return OR_BAD_DTYPE;
  if (M < 0 || K < 1 || N < 1 || ldx < K || ldy < N) return OR_BAD_SHAPE;
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; ++m) {
    for (int n = 0; n < N; ++n) {
      double s = 0.0;
      for (int k = 0; k < K; ++k)
        s += load_elem(x, x_dtype, (size_t)m * ldx + k) * load_elem(w, w_dtype, (size_t)n * K + k);
      if (bias) s += (double)bias[n];
      if (relu && !(s > 0.0)) s = 0.0;
      store_elem(y, y_dtype, (size_t)m * ldy + n, s);
    }
  }
  return OR_OK;
}

/*
 * Backward of one dense layer, given dz = dL/d(pre-activation) [M][N] (stride ldz):
 *   dx[m][k] = sum_n dz[m][n] * w[n][k]         (times 1[xmask[m][k] > 0] when xmask is given:
 *                                                 the ReLU of the layer below, whose output
 *                                                 x is; this makes dx the dz of that layer)
 *   dw[n][k] = sum_m dz[m][n] * x[m][k]
 *   db[n]    = sum_m dz[m][n]
 * dx (stride ldx) may be NULL (first layer).  Sums in double, ascending index order, one
 * rounding per output.
 */
int oracle_linear_bwd(const void* x, int x_dtype, int M, int K, int ldx, const void* w,
                      int w_dtype, int N, const void* dz, int dz_dtype, int ldz,
                      const void* xmask, void* dx, int dx_dtype, void* dw, void* db,
                      int wgrad_dtype) {
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype) || !dtype_ok(dz_dtype) || !dtype_ok(dx_dtype) ||
      !dtype_ok(wgrad_dtype))
    return OR_BAD_DTYPE;
  if (M < 0 || K < 1 || N < 1 || ldx < K || ldz < N) return OR_BAD_SHAPE;
  if (dx) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
      for (int k = 0; k < K; ++k) {
        double s = 0.0;
        for (int n = 0; n < N; ++n)
          s += load_elem(dz, dz_dtype, (size_t)m * ldz + n) * load_elem(w, w_dtype, (size_t)n * K + k);
        if (xmask && !(load_elem(xmask, x_dtype, (size_t)m * ldx + k) > 0.0)) s = 0.0;
        store_elem(dx, dx_dtype, (size_t)m * ldx + k, s);
      }
    }
  }
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    for (int k = 0; k < K; ++k) {
      double s = 0.0;
      for (int m = 0; m < M; ++m)
        s += load_elem(dz, dz_dtype, (size_t)m * ldz + n) * load_elem(x, x_dtype, (size_t)m * ldx + k);
      store_elem(dw, wgrad_dtype, (size_t)n * K + k, s);
    }
    double s = 0.0;
    for (int m = 0; m < M; ++m) s += load_elem(dz, dz_dtype, (size_t)m * ldz + n);
    store_elem(db, wgrad_dtype, (size_t)n, s);
  }
  return OR_OK;
}

/*
 * Backward of a ReLU given its output y:  dz[m][n] = dy[m][n] * 1[y[m][n] > 0]  (all three
 * [M] rows of stride ld, first N used).
 */
int oracle_relu_bwd(const void* dy, const void* y, int dtype, int M, int N, int ld, void* dz) {
  if (!dtype_ok(dtype)) return OR_BAD_DTYPE;
  if (M < 0 || N < 1 || ld < N) return OR_BAD_SHAPE;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      size_t i = (size_t)m * ld + n;
      store_elem(dz, dtype, i, load_elem(y, dtype, i) > 0.0 ? load_elem(dy, dtype, i) : 0.0);
    }
  return OR_OK;
}

/*
 * Logistic loss on one logit per sample, label y in {0, 1} (fp32):
 *   loss = (1/M) sum_m [ max(z,0) - z*y + log(1 + exp(-|z|)) ]      (= -log p or -log(1-p),
 *                                                                     p = 1/(1+exp(-z)))
 *   dz[m] = (p_m - y_m) / M
 * `loss` receives the double value; dz is rounded once to dz_dtype.
 */
int oracle_bce_logits(const void* z, int z_dtype, const float* labels, int M, double* loss,
                      void* dz, int dz_dtype) {
  if (!dtype_ok(z_dtype) || !dtype_ok(dz_dtype)) return OR_BAD_DTYPE;
  if (M < 1) return OR_BAD_SHAPE;
  double s = 0.0;
  for (int m = 0; m < M; ++m) {
    double v = load_elem(z, z_dtype, (size_t)m), y = (double)labels[m];
    s += (v > 0.0 ? v : 0.0) - v * y + log1p(exp(-fabs(v)));
    double p = 1.0 / (1.0 + exp(-v));
    store_elem(dz, dz_dtype, (size_t)m, (p - y) / (double)M);
  }
  *loss = s / (double)M;
  return OR_OK;
}

/*
 * Plain SGD on a dense parameter kept in fp32 (the page keeps the MLPs in mixed precision:
 * an fp32 master copy, a 16-bit copy for the products):
 *   master[i] <- round_f32( master[i] - lr * grad[i] ),   copy[i] <- round_copy( master[i] )
 * copy may be NULL.
 */
int oracle_sgd_dense(float* master, const float* grad, int64_t n, float lr, void* copy,
                     int copy_dtype) {
  if (copy && !dtype_ok(copy_dtype)) return OR_BAD_DTYPE;
  for (int64_t i = 0; i < n; ++i) {
    master[i] = (float)((double)master[i] - (double)lr * (double)grad[i]);
    if (copy) store_elem(copy, copy_dtype, (size_t)i, (double)master[i]);
  }
  return OR_OK;
}

int oracle_version(void) { return 3; }
