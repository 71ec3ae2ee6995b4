/*
 * Every entry point of the CPU oracle on small inputs, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure; CPU only).
 *
 * Buffers are allocated at their exact extent (strided rows end at the last element used),
 * so a read or write one element past what the oracle's documented layout allows is
 * reported; shapes are odd (D = 5, strides above the row length), bags are empty, single
 * and long, indices negative and oversize under hashing, and the error paths (bad index,
 * bad offsets, bad dtype, bad shape) are taken once each.  The program prints "ok" and
 * exits 0 when every call returned the expected status; a sanitizer finding aborts it.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/emb_oracle.c"

static int failures = 0;

#define EXPECT(call, want)                                                          \
  do {                                                                              \
    int rc_ = (call);                                                               \
    if (rc_ != (want)) {                                                            \
      printf("FAIL line %d: %s returned %d, expected %d\n", __LINE__, #call, rc_, (want)); \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

static size_t esize(int dtype) {
  switch (dtype) {
    case OR_F32: return 4;
    case OR_F64: return 8;
    default: return 2;
  }
}

static uint32_t lcg = 12345u;
static double next_value(void) {
  lcg = lcg * 1664525u + 1013904223u;
  return ((double)(lcg >> 8) / (double)(1u << 24)) * 2.0 - 1.0;  /* [-1, 1) */
}

/* n elements of dtype, filled with values in [-1, 1) rounded to the dtype */
static void* filled(size_t n, int dtype) {
  void* p = malloc(n ? n * esize(dtype) : 1);
  for (size_t i = 0; i < n; ++i) store_elem(p, dtype, i, next_value());
  return p;
}

static const int kDtypes[4] = {OR_F32, OR_F16, OR_BF16, OR_F64};

static void bag_and_update(void) {
  /* three tables of 3, 1 and 7 rows; B = 4; bag lengths 0, 1, 3, 2, ... */
  const int F = 3, B = 4, D = 5;
  const int64_t row_offset[4] = {0, 3, 4, 11};
  const int32_t offsets[13] = {0, 0, 1, 4, 6, 7, 7, 8, 9, 12, 12, 13, 15};
  /* valid local rows for the plain run */
  const int32_t idx_ok[15] = {2, 0, 1, 2, 1, 1, 0, 0, 0, 6, 3, 6, 5, 0, 4};
  /* negative and oversize, for the floor-modulo run */
  const int32_t idx_hash[15] = {-1, 5, -7, 2, 100, -2, 3, -1, 9, -8, 13, 6, 2147483647, -2147483647 - 1, 4};
  const int32_t idx_bad[15] = {2, 0, 1, 3, 1, 1, 0, 0, 0, 6, 3, 6, 5, 0, 4}; /* 3 >= rows of table 0 */
  const int32_t offsets_bad[13] = {0, 0, 1, 4, 6, 7, 7, 8, 9, 12, 12, 11, 15};
  const int64_t nnz = 15;
  for (int wt = 0; wt < 4; ++wt) {
    for (int ot = 0; ot < 4; ++ot) {
      void* W = filled((size_t)row_offset[F] * D, kDtypes[wt]);
      void* out = malloc((size_t)B * F * D * esize(kDtypes[ot]));
      EXPECT(oracle_emb_bag_fwd(W, kDtypes[wt], row_offset, F, D, idx_ok, offsets, B, 0, out, kDtypes[ot]), OR_OK);
      EXPECT(oracle_emb_bag_fwd(W, kDtypes[wt], row_offset, F, D, idx_hash, offsets, B, 1, out, kDtypes[ot]), OR_OK);
      EXPECT(oracle_emb_bag_fwd(W, kDtypes[wt], row_offset, F, D, idx_bad, offsets, B, 0, out, kDtypes[ot]),
             OR_BAD_INDEX);
      EXPECT(oracle_emb_bag_fwd(W, kDtypes[wt], row_offset, F, D, idx_ok, offsets_bad, B, 0, out, kDtypes[ot]),
             OR_BAD_OFFSETS);
      EXPECT(oracle_emb_bag_fwd(W, 7, row_offset, F, D, idx_ok, offsets, B, 0, out, kDtypes[ot]), OR_BAD_DTYPE);
      void* demb = filled((size_t)B * F * D, kDtypes[ot]);
      EXPECT(oracle_grad_reduce_update(W, kDtypes[wt], row_offset, F, D, idx_ok, offsets, B, 0, demb, kDtypes[ot],
                                       0.25f), OR_OK);
      EXPECT(oracle_grad_reduce_update(W, kDtypes[wt], row_offset, F, D, idx_hash, offsets, B, 1, demb,
                                       kDtypes[ot], 0.25f), OR_OK);
      EXPECT(oracle_grad_reduce_update(W, kDtypes[wt], row_offset, F, D, idx_bad, offsets, B, 0, demb, kDtypes[ot],
                                       0.25f), OR_BAD_INDEX);
      free(demb);
      free(out);
      free(W);
    }
  }
  /* the sort: outputs of exactly nnz entries, nnz + 1 segment offsets */
  uint32_t* rows = malloc(nnz * sizeof(uint32_t));
  uint32_t* bags = malloc(nnz * sizeof(uint32_t));
  uint32_t* uniq = malloc(nnz * sizeof(uint32_t));
  uint32_t* segs = malloc((nnz + 1) * sizeof(uint32_t));
  uint32_t nu = 0;
  EXPECT(oracle_grad_sort(row_offset, F, idx_ok, offsets, B, 0, rows, bags, uniq, segs, &nu), OR_OK);
  EXPECT(oracle_grad_sort(row_offset, F, idx_hash, offsets, B, 1, rows, bags, uniq, segs, &nu), OR_OK);
  EXPECT(oracle_grad_sort(row_offset, F, idx_bad, offsets, B, 0, rows, bags, uniq, segs, &nu), OR_BAD_INDEX);
  /* every lookup of one row: a single segment */
  const int32_t idx_same[15] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  EXPECT(oracle_grad_sort(row_offset, F, idx_same, offsets, B, 0, rows, bags, uniq, segs, &nu), OR_OK);
  if (nu != 3) { printf("FAIL: %u segments for one row per table\n", nu); ++failures; }
  free(rows); free(bags); free(uniq); free(segs);
  /* an empty batch */
  const int32_t off0[1] = {0};
  void* W = filled((size_t)row_offset[F] * D, OR_F32);
  EXPECT(oracle_emb_bag_fwd(W, OR_F32, row_offset, 1, D, idx_ok, off0, 0, 0, W, OR_F32), OR_OK);
  EXPECT(oracle_emb_bag_fwd(W, OR_F32, row_offset, 0, D, idx_ok, off0, 0, 0, W, OR_F32), OR_BAD_SHAPE);
  free(W);
}

static void interactions(void) {
  const int B = 3, F = 3, D = 5, V = F + 1, P = V * (V - 1) / 2;
  for (int it = 0; it < 4; ++it) {
    for (int ot = 0; ot < 4; ++ot) {
      for (int pad = 0; pad <= 5; pad += 5) {
        const int S = D + P + pad;
        void* x0 = filled((size_t)B * D, kDtypes[it]);
        void* emb = filled((size_t)B * F * D, kDtypes[it]);
        void* out = malloc((size_t)B * S * esize(kDtypes[ot]));
        EXPECT(oracle_dot_interact_fwd(x0, emb, kDtypes[it], B, F, D, out, kDtypes[ot], S), OR_OK);
        void* dout = filled((size_t)B * S, kDtypes[ot]);
        void* dx0 = malloc((size_t)B * D * esize(kDtypes[it]));
        void* demb = malloc((size_t)B * F * D * esize(kDtypes[it]));
        EXPECT(oracle_dot_interact_bwd(x0, emb, kDtypes[it], B, F, D, dout, kDtypes[ot], S, dx0, demb, kDtypes[it]),
               OR_OK);
        free(out); free(dout);
        const int SC = V * D + pad;
        out = malloc((size_t)B * SC * esize(kDtypes[ot]));
        EXPECT(oracle_cat_interact_fwd(x0, emb, kDtypes[it], B, F, D, out, kDtypes[ot], SC), OR_OK);
        dout = filled((size_t)B * SC, kDtypes[ot]);
        EXPECT(oracle_cat_interact_bwd(dout, kDtypes[ot], B, F, D, SC, dx0, demb, kDtypes[it]), OR_OK);
        free(out); free(dout); free(x0); free(emb); free(dx0); free(demb);
      }
    }
  }
  void* x0 = filled((size_t)B * D, OR_F32);
  void* emb = filled((size_t)B * F * D, OR_F32);
  void* out = malloc((size_t)B * (D + P) * 4);
  EXPECT(oracle_dot_interact_fwd(x0, emb, OR_F32, B, F, D, out, OR_F32, D + P - 1), OR_BAD_SHAPE);
  EXPECT(oracle_dot_interact_fwd(x0, emb, 9, B, F, D, out, OR_F32, D + P), OR_BAD_DTYPE);
  free(x0); free(emb); free(out);
}

static void dense(void) {
  const int M = 5, K = 7, N = 3, ldx = 9, ldy = 4;
  const size_t nx = (size_t)(M - 1) * ldx + K, ny = (size_t)(M - 1) * ldy + N;
  for (int t = 0; t < 4; ++t) {
    const int dt = kDtypes[t];
    void* x = filled(nx, dt);
    void* w = filled((size_t)N * K, dt);
    float* bias = malloc(N * sizeof(float));
    for (int n = 0; n < N; ++n) bias[n] = (float)next_value();
    void* y = malloc(ny * esize(dt));
    EXPECT(oracle_linear_fwd(x, dt, M, K, ldx, w, dt, N, bias, 1, y, dt, ldy), OR_OK);
    EXPECT(oracle_linear_fwd(x, dt, M, K, ldx, w, dt, N, NULL, 0, y, dt, ldy), OR_OK);
    EXPECT(oracle_linear_fwd(x, dt, 0, K, ldx, w, dt, N, bias, 1, y, dt, ldy), OR_OK);
    EXPECT(oracle_linear_fwd(x, dt, M, K, K - 1, w, dt, N, bias, 1, y, dt, ldy), OR_BAD_SHAPE);
    void* dz = filled(ny, dt);
    void* dx = malloc(nx * esize(dt));
    void* dw = malloc((size_t)N * K * 4);
    void* db = malloc((size_t)N * 4);
    EXPECT(oracle_linear_bwd(x, dt, M, K, ldx, w, dt, N, dz, dt, ldy, x, dx, dt, dw, db, OR_F32), OR_OK);
    EXPECT(oracle_linear_bwd(x, dt, M, K, ldx, w, dt, N, dz, dt, ldy, NULL, NULL, dt, dw, db, OR_F32), OR_OK);
    EXPECT(oracle_linear_bwd(x, dt, 0, K, ldx, w, dt, N, dz, dt, ldy, NULL, dx, dt, dw, db, OR_F32), OR_OK);
    void* dz2 = malloc(ny * esize(dt));
    EXPECT(oracle_relu_bwd(dz, y, dt, M, N, ldy, dz2), OR_OK);
    EXPECT(oracle_relu_bwd(dz, y, dt, M, N, N - 1, dz2), OR_BAD_SHAPE);
    free(dz2); free(dz); free(dx); free(dw); free(db); free(y); free(bias); free(w); free(x);
  }
  /* loss and dense SGD */
  void* z = filled(M, OR_BF16);
  float* labels = malloc(M * sizeof(float));
  for (int m = 0; m < M; ++m) labels[m] = (float)(m % 2);
  void* dzl = malloc(M * 2);
  double loss = 0.0;
  EXPECT(oracle_bce_logits(z, OR_BF16, labels, M, &loss, dzl, OR_BF16), OR_OK);
  EXPECT(oracle_bce_logits(z, OR_BF16, labels, 0, &loss, dzl, OR_BF16), OR_BAD_SHAPE);
  free(z); free(labels); free(dzl);
  const int64_t n = 11;
  float* master = malloc(n * sizeof(float));
  float* grad = malloc(n * sizeof(float));
  for (int64_t i = 0; i < n; ++i) { master[i] = (float)next_value(); grad[i] = (float)next_value(); }
  for (int t = 0; t < 4; ++t) {
    void* copy = malloc((size_t)n * esize(kDtypes[t]));
    EXPECT(oracle_sgd_dense(master, grad, n, 0.5f, copy, kDtypes[t]), OR_OK);
    free(copy);
  }
  EXPECT(oracle_sgd_dense(master, grad, n, 0.5f, NULL, OR_F32), OR_OK);
  free(master); free(grad);
  /* the converters' array forms */
  double* xd = malloc(n * sizeof(double));
  for (int64_t i = 0; i < n; ++i) xd[i] = next_value() * 1e5;
  for (int t = 0; t < 4; ++t) {
    void* r = malloc((size_t)n * esize(kDtypes[t]));
    oracle_round_f64(xd, n, kDtypes[t], r);
    oracle_widen(r, n, kDtypes[t], xd);
    free(r);
  }
  free(xd);
}

int main(void) {
  bag_and_update();
  interactions();
  dense();
  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
