"""The oracle's pins must reject plausible mistakes (CPU only).

Each case copies the oracle's C source, plants one mistake (a wrong sign, a dropped term,
a transposed index, a wrong pair order, a broken tie-break, a broken rounding), builds it
into a temporary library and runs the pin battery of ``test_oracle_pins`` against it.  At
least one pin must fail for every planted mistake.  The shipped oracle is untouched.
"""
import os
import subprocess
import tempfile

import pytest

from oracle import build as obuild
from oracle import oracle as orc
from tests import test_oracle_pins as pins

MUTANTS = [
    ("pooling sign", "acc[d] = (k == offsets[g]) ? w : acc[d] + w;", "acc[d] = (k == offsets[g]) ? w : acc[d] - w;"),
    ("pooling starts from +0", "acc[d] = (k == offsets[g]) ? w : acc[d] + w;", "acc[d] = acc[d] + w;"),
    ("pooled output transposed", "store_elem(out, out_dtype, ((size_t)b * F + t) * D + d, acc[d]);",
     "store_elem(out, out_dtype, ((size_t)t * B + b) * D + d, acc[d]);"),
    ("C remainder instead of floor modulo", "return r < 0 ? r + n : r;", "return r;"),
    ("pair order reversed within a row", "return (int64_t)i * (i - 1) / 2 + j;",
     "return (int64_t)i * (i - 1) / 2 + (i - 1 - j);"),
    ("dropped first term of a dot product",
     "for (int d = 0; d < D; ++d)\n          s += vec_elem",
     "for (int d = 1; d < D; ++d)\n          s += vec_elem"),
    ("wrong operand in the backward product",
     "acc += s * vec_elem(x0, emb, in_dtype, b, F, D, j, d);",
     "acc += s * vec_elem(x0, emb, in_dtype, b, F, D, k, d);"),
    ("dx0 misses the direct term",
     "load_elem(dout, dout_dtype, row + d) + acc);", "acc);"),
    ("unstable tie order", "if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;",
     "if (x->pos != y->pos) return x->pos < y->pos ? 1 : -1;"),
    ("SGD sign", "load_elem(W, w_dtype, i) - (double)lr * acc[d]",
     "load_elem(W, w_dtype, i) + (double)lr * acc[d]"),
    ("truncating instead of rounding", "double r = nearbyint(n) * quantum;",
     "double r = floor(n) * quantum;"),
    ("subnormal quantum not clamped", "if (E < emin) E = emin;", ""),
    ("padding not zeroed", "for (int64_t c = D + P; c < out_stride; ++c) store_elem(out, out_dtype, row + c, 0.0);", ""),
    ("cat blocks in the wrong order",
     "store_elem(out, out_dtype, row + (size_t)v * D + d, vec_elem(x0, emb, in_dtype, b, F, D, v, d));",
     "store_elem(out, out_dtype, row + (size_t)v * D + d, vec_elem(x0, emb, in_dtype, b, F, D, (v + 1) % V, d));"),
    ("cat padding not zeroed",
     "for (int64_t c = (int64_t)V * D; c < out_stride; ++c) store_elem(out, out_dtype, row + c, 0.0);", ""),
    ("cat gradient read from the neighbouring block",
     "load_elem(dout, dout_dtype, row + (size_t)(1 + t) * D + d));",
     "load_elem(dout, dout_dtype, row + (size_t)t * D + d));"),
    ("cat gradient with tables and dimensions transposed",
     "store_elem(demb, grad_dtype, ((size_t)b * F + t) * D + d,",
     "store_elem(demb, grad_dtype, ((size_t)b * D + d) * F + t,"),
    ("dense layer reads its weights transposed",
     "s += load_elem(x, x_dtype, (size_t)m * ldx + k) * load_elem(w, w_dtype, (size_t)n * K + k);",
     "s += load_elem(x, x_dtype, (size_t)m * ldx + k) * load_elem(w, w_dtype, ((size_t)k * N + n) % ((size_t)N * K));"),
    ("dense layer drops its bias", "if (bias) s += (double)bias[n];", ""),
    ("ReLU not applied", "if (relu && !(s > 0.0)) s = 0.0;", ""),
    ("input gradient without the ReLU mask",
     "if (xmask && !(load_elem(xmask, x_dtype, (size_t)m * ldx + k) > 0.0)) s = 0.0;", ""),
    ("weight gradient pairs dz with the wrong sample",
     "s += load_elem(dz, dz_dtype, (size_t)m * ldz + n) * load_elem(x, x_dtype, (size_t)m * ldx + k);",
     "s += load_elem(dz, dz_dtype, (size_t)m * ldz + n) * load_elem(x, x_dtype, (size_t)((m + 1) % M) * ldx + k);"),
    ("bias gradient sums one column", "for (int m = 0; m < M; ++m) s += load_elem(dz, dz_dtype, (size_t)m * ldz + n);",
     "for (int m = 0; m < M; ++m) s += load_elem(dz, dz_dtype, (size_t)m * ldz);"),
    ("logistic gradient sign", "store_elem(dz, dz_dtype, (size_t)m, (p - y) / (double)M);",
     "store_elem(dz, dz_dtype, (size_t)m, (y - p) / (double)M);"),
    ("ReLU backward passes gradients at y = 0",
     "store_elem(dz, dtype, i, load_elem(y, dtype, i) > 0.0 ? load_elem(dy, dtype, i) : 0.0);",
     "store_elem(dz, dtype, i, load_elem(y, dtype, i) >= 0.0 ? load_elem(dy, dtype, i) : 0.0);"),
    ("loss not averaged", "*loss = s / (double)M;", "*loss = s;"),
    ("dense SGD sign", "master[i] = (float)((double)master[i] - (double)lr * (double)grad[i]);",
     "master[i] = (float)((double)master[i] + (double)lr * (double)grad[i]);"),
]


def battery():
    """Every pin of test_oracle_pins, with fixed parameters."""
    return [
        pins.test_f32_to_f16_matches_numpy,
        pins.test_f64_to_f16_direct_matches_numpy,
        pins.test_f32_to_bf16_matches_torch,
        pins.test_f64_to_bf16_direct_bruteforce,
        pins.test_bf16_overflow_and_f32_store,
        lambda: pins.test_emb_bag_equals_dense_count_matrix("f64"),
        lambda: pins.test_emb_bag_equals_dense_count_matrix("bf16"),
        pins.test_emb_bag_hotness1_is_index_select_bit_exact,
        pins.test_emb_bag_empty_bags_give_positive_zero,
        pins.test_emb_bag_hotness1_keeps_signed_zeros_and_subnormals,
        pins.test_emb_bag_hash_is_floor_modulo,
        pins.test_emb_bag_rounding_is_single_rne,
        lambda: pins.test_dot_fwd_equals_masked_gram(8, 16),
        pins.test_dot_fwd_two_vectors_is_one_dot_product,
        pins.test_dot_fwd_pair_sum_closed_form,
        lambda: pins.test_dot_bwd_central_differences_exact_for_quadratic(3, 4),
        pins.test_dot_bwd_matches_symmetric_matrix_product_and_euler,
        lambda: pins.test_cat_fwd_equals_numpy_stack_of_the_vectors(8, 16, 5),
        pins.test_cat_fwd_blocks_are_the_vectors_the_dot_interaction_multiplies,
        pins.test_cat_fwd_bf16_is_an_exact_copy_and_f32_narrowing_rounds_once,
        pins.test_cat_bwd_central_differences_and_adjoint_identity,
        pins.test_cat_bwd_of_the_forward_output_returns_the_inputs_and_ignores_padding,
        lambda: pins.test_grad_sort_matches_numpy_stable_argsort(True),
        pins.test_grad_sort_counting_sort_on_tiny_key_range,
        lambda: pins.test_grad_update_equals_dense_sgd(5),
        pins.test_grad_update_invariants,
        pins.test_grad_update_single_repeated_row_is_column_sum,
        lambda: pins.test_linear_fwd_matches_float64_matmul_on_exact_values(True),
        pins.test_linear_fwd_respects_row_strides,
        pins.test_linear_bwd_central_differences_exact,
        pins.test_linear_bwd_mask_is_the_relu_derivative,
        pins.test_linear_bwd_transposition_identity,
        pins.test_bce_closed_forms,
        pins.test_bce_gradient_central_differences,
        pins.test_sgd_dense_special_cases,
        pins.test_mlp_chain_gradient_central_differences,
        pins.test_relu_bwd_is_the_relu_derivative,
    ]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        csrc = os.path.join(tmp, "mutant.c")
        so = os.path.join(tmp, "libmutant.so")
        open(csrc, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                        "-o", so, csrc, "-lm"], check=True)
        prev = orc.use_library(so)
        failed = []
        try:
            for check in battery():
                try:
                    check()
                except (AssertionError, ValueError):
                    failed.append(check)
        finally:
            orc.restore_library(prev)
    assert failed, f"no pin rejects the planted mistake '{name}'"
