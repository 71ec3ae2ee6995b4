"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test states what fixes the expected value:
  - library routines (numpy's binary16 conversion, torch's bfloat16 conversion, numpy's
    stable argsort, float64 matmul),
  - brute force on tiny inputs (dense count matrices, an exhaustive nearest-value search),
  - closed forms and invariants of the interaction (sum of pairs, Euler's identity for a
    quadratic form, exactness of central differences on a quadratic),
  - special cases (hotness 1 is an index select, two vectors give one dot product, one
    repeated row gives one segment, lr = 0 leaves the tables unchanged).

The definitions pinned are those of the page "DLRM For PyTorch", §Model architecture
(embedding per categorical feature, dot interaction, concatenation with the bottom-MLP
output) and §Command-line options (--hash_indices, --lr).
"""

import numpy as np
import pytest
import torch

from oracle import oracle as orc

RNG = np.random.default_rng(20240611)
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ----------------------------------------------------------------------------------------
# helpers (independent of the oracle)
# ----------------------------------------------------------------------------------------

def bf16_bits_to_f64_torch(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.astype(np.int32).astype(np.int16)).view(torch.bfloat16).double().numpy()


def f32_to_bf16_bits_torch(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


_ALL_BF16 = None


def _bf16_table():
    """All finite bf16 values, as float64, sorted; with their bit patterns."""
    global _ALL_BF16
    if _ALL_BF16 is None:
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        vals = bf16_bits_to_f64_torch(bits)
        ok = np.isfinite(vals)
        bits, vals = bits[ok], vals[ok]
        # drop -0 so each value appears once (+0 kept)
        keep = ~((vals == 0) & (bits == 0x8000))
        bits, vals = bits[keep], vals[keep]
        order = np.argsort(vals, kind="stable")
        _ALL_BF16 = (vals[order], bits[order])
    return _ALL_BF16


def nearest_bf16_bruteforce(x: float) -> int:
    """Exhaustive search: the finite bf16 value closest to x, ties to the even pattern."""
    vals, bits = _bf16_table()
    d = np.abs(vals - x)
    m = d.min()
    cand = np.nonzero(d == m)[0]
    if cand.size > 1:
        even = [c for c in cand if bits[c] % 2 == 0]
        c = even[0]
    else:
        c = cand[0]
    b = int(bits[c])
    if b == 0 and np.signbit(x):
        b = 0x8000
    return b


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref * ref)) if ref.size else 1.0)
    scale = np.where(scale == 0, 1.0, scale)
    return float(np.max(np.abs(got - ref) / scale)) if ref.size else 0.0


def make_problem(rng, F, B, rows, D, lengths="one", hash_range=False):
    rows = list(rows)
    row_offset = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    if lengths == "one":
        lens = np.ones((F, B), np.int64)
    else:
        lens = rng.integers(0, lengths + 1, size=(F, B))
    offsets = np.concatenate([[0], np.cumsum(lens.reshape(-1))]).astype(np.int32)
    idx = []
    for t in range(F):
        n = int(lens[t].sum())
        if hash_range:
            idx.append(rng.integers(-3 * rows[t], 3 * rows[t], size=n))
        else:
            idx.append(rng.integers(0, rows[t], size=n))
    indices = np.concatenate(idx).astype(np.int32) if idx else np.zeros(0, np.int32)
    return row_offset, offsets, indices


def dense_counts(row_offset, offsets, indices, B, t):
    """Brute force: A[b, r] = number of times row r of table t occurs in bag (t, b)."""
    n = int(row_offset[t + 1] - row_offset[t])
    A = np.zeros((B, n), np.float64)
    for b in range(B):
        g = t * B + b
        for k in range(offsets[g], offsets[g + 1]):
            A[b, int(indices[k]) % n] += 1.0  # python % = floor modulo
    return A


# ----------------------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------------------

def _fp32_patterns(n_low=96):
    """All 2^16 high halves x a set of low halves (ties, neighbours of ties, random)."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x0FFF, 0x1000, 0x1001,
            0x2000, 0x3000, 0x6000, 0x7000, 0xF000, 0xE000, 0x5000]
    lows += list(RNG.integers(0, 65536, size=n_low - len(lows)))
    lows = np.array(lows, np.uint32)
    return (hi[:, None] | lows[None, :]).reshape(-1)


def test_f32_to_f16_matches_numpy():
    bits = _fp32_patterns()
    x = bits.view(np.float32)
    ours = orc.round_from_f64(x.astype(np.float64), "f16")
    ref = x.astype(np.float16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours[~nan].astype(np.float64)), np.zeros((~nan).sum(), bool))
    assert np.array_equal(ours.view(np.uint16)[~nan], ref.view(np.uint16)[~nan])
    assert np.all(np.isnan(ours[nan]))


def test_f64_to_f16_direct_matches_numpy():
    # doubles just above / below binary16 ties, in the normal and the subnormal range
    base = np.concatenate([RNG.uniform(-70000, 70000, 4000), RNG.uniform(-1e-4, 1e-4, 4000)])
    h = base.astype(np.float16).astype(np.float64)
    ulp = np.abs(np.spacing(base.astype(np.float16)).astype(np.float64))
    ties = h + ulp / 2
    x = np.concatenate([base, ties, ties + 1e-12 * np.abs(ties) + 1e-30, ties - 1e-12 * np.abs(ties) - 1e-30,
                        [65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 2.0**-24, 2.0**-25,
                         2.0**-25 * 1.0000001, 3 * 2.0**-26, 0.0, -0.0]])
    x = x[np.isfinite(x)]
    ours = orc.round_from_f64(x, "f16")
    ref = x.astype(np.float16)
    assert np.array_equal(ours.view(np.uint16), ref.view(np.uint16))


def test_f32_to_bf16_matches_torch():
    bits = _fp32_patterns()
    x = bits.view(np.float32)
    ours = orc.round_from_f64(x.astype(np.float64), "bf16")
    ref = f32_to_bf16_bits_torch(x)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN (quiet), sign kept
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


def test_f64_to_bf16_direct_bruteforce():
    # doubles that round differently directly and through binary32 (double rounding)
    xs = []
    for _ in range(150):
        m = RNG.integers(128, 256)
        e = int(RNG.integers(-130, 110))
        tie = (m + 0.5) * 2.0**e
        xs += [tie, tie * (1 + 2.0**-40), tie * (1 - 2.0**-40), m * 2.0**e * (1 + RNG.uniform(0, 2**-7))]
    xs += [1 + 2.0**-8 + 2.0**-40, -(1 + 2.0**-8 + 2.0**-40), 2.0**-133, 2.0**-134, 3 * 2.0**-135]
    xs = np.array(xs)
    ours = orc.round_from_f64(xs, "bf16")
    for x, o in zip(xs, ours):
        assert int(o) == nearest_bf16_bruteforce(float(x)), (x, hex(int(o)))


def test_bf16_overflow_and_f32_store():
    big = np.array([3.4e38, 3.39e38, 1e39, -1e39, np.inf, -np.inf])
    ours = orc.round_from_f64(big, "bf16")
    assert ours[2] == 0x7F80 and ours[3] == 0xFF80 and ours[4] == 0x7F80 and ours[5] == 0xFF80
    x = np.concatenate([RNG.normal(size=1000), RNG.normal(size=1000) * 1e-40, [1e39]])
    assert np.array_equal(orc.round_from_f64(x, "f32").view(np.uint32), x.astype(np.float32).view(np.uint32))


def test_converters_exhaustive_over_all_fp32_patterns(tmp_path):
    """All 2^32 binary32 patterns through the oracle's bf16 and fp16 rounding, against the
    x86 F16C conversion (binary16) and round-to-nearest-even on the bit pattern (bfloat16);
    the C program is tests/native/p4_converters.c (OpenMP, about 20 s on 8 cores)."""
    import os
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    with open("/proc/cpuinfo") as f:
        if "f16c" not in f.read():
            pytest.skip("the host CPU has no F16C conversion instructions")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "p4_converters.c")
    exe = str(tmp_path / "p4_converters")
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-mf16c", "-ffp-contract=off",
                    "-Wno-unknown-pragmas", "-o", exe, src, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bf16 mismatches 0" in r.stdout and "f16 mismatches 0" in r.stdout


def test_widening_is_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = orc.widen(bits, "bf16")
    ref = bf16_bits_to_f64_torch(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(w[ok], ref[ok]) and np.all(np.isnan(w[~ok]))
    h = bits.view(np.float16)
    w = orc.widen(h, "f16")
    ref = h.astype(np.float64)
    ok = ~np.isnan(ref)
    assert np.array_equal(w[ok], ref[ok]) and np.all(np.isnan(w[~ok]))


# ----------------------------------------------------------------------------------------
# embedding bag forward
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("w_dtype", ["f64", "f32", "bf16", "f16"])
def test_emb_bag_equals_dense_count_matrix(w_dtype):
    rng = np.random.default_rng(1)
    F, B, D = 3, 7, 5
    rows = [11, 4, 9]
    row_offset, offsets, indices = make_problem(rng, F, B, rows, D, lengths=6)
    Wd = rng.normal(0, 0.5, size=(sum(rows), D))
    W = orc.round_from_f64(Wd, w_dtype)
    Wexact = orc.widen(W, w_dtype) if w_dtype != "f64" else W
    out = orc.emb_bag_fwd(W, w_dtype, row_offset, indices, offsets, B, D, "f64")
    for t in range(F):
        A = dense_counts(row_offset, offsets, indices, B, t)
        ref = A @ Wexact[row_offset[t]:row_offset[t + 1]]
        np.testing.assert_allclose(out[:, t, :], ref, rtol=1e-13, atol=1e-15)


def test_emb_bag_hotness1_is_index_select_bit_exact():
    rng = np.random.default_rng(2)
    F, B, D = 4, 33, 16
    rows = [50, 1, 7, 20]
    row_offset, offsets, indices = make_problem(rng, F, B, rows, D)
    W = rng.normal(0, 0.01, size=(sum(rows), D)).astype(np.float32)
    out32 = orc.emb_bag_fwd(W, "f32", row_offset, indices, offsets, B, D, "f32")
    out16 = orc.emb_bag_fwd(W, "f32", row_offset, indices, offsets, B, D, "bf16")
    for t in range(F):
        sel = W[row_offset[t] + indices[t * B:(t + 1) * B]]
        assert np.array_equal(out32[:, t, :].view(np.uint32), sel.view(np.uint32))
        assert np.array_equal(out16[:, t, :], f32_to_bf16_bits_torch(sel))


def test_emb_bag_hotness1_keeps_signed_zeros_and_subnormals():
    # a one-row bag is an index select: -0.0 and fp16 subnormal rows come back bit for bit
    F, B, D = 1, 4, 8
    row_offset = np.array([0, 4], np.int64)
    offsets = np.arange(B + 1, dtype=np.int32)
    indices = np.array([0, 1, 2, 3], np.int32)
    bits = np.array([[0x8000] * 8, [0x0001] * 8, [0x8001] * 8, [0x03FF] * 8], np.uint16)
    W = bits.view(np.float16)
    out = orc.emb_bag_fwd(W, "f16", row_offset, indices, offsets, B, D, "f16")
    assert np.array_equal(out.view(np.uint16).reshape(B, D), bits)
    out32 = orc.emb_bag_fwd(W, "f16", row_offset, indices, offsets, B, D, "f32")
    assert np.array_equal(out32.reshape(B, D), W.astype(np.float32))
    assert np.signbit(out32[0, 0, 0])


def test_emb_bag_empty_bags_give_positive_zero():
    F, B, D = 2, 3, 4
    row_offset = np.array([0, 5, 10], np.int64)
    offsets = np.array([0, 0, 1, 1, 1, 2, 2], np.int32)  # bags g = 0, 2, 3, 5 empty
    indices = np.array([3, 4], np.int32)
    W = -np.ones((10, D), np.float32)
    out = orc.emb_bag_fwd(W, "f32", row_offset, indices, offsets, B, D, "f32")
    assert np.all(out[1, 0] == -1) and np.all(out[1, 1] == -1)  # g = 1 and g = 4
    for b, t in ((0, 0), (2, 0), (0, 1), (2, 1)):
        assert np.array_equal(out[b, t].view(np.uint32), np.zeros(D, np.uint32))


def test_emb_bag_hash_is_floor_modulo():
    rng = np.random.default_rng(3)
    F, B, D = 3, 10, 3
    rows = [7, 13, 5]
    row_offset, offsets, indices = make_problem(rng, F, B, rows, D, lengths=3, hash_range=True)
    W = rng.normal(size=(sum(rows), D))
    hashed = orc.emb_bag_fwd(W, "f64", row_offset, indices, offsets, B, D, "f64", hash_indices=True)
    modded = indices.copy().astype(np.int64)
    for t in range(F):
        s, e = offsets[t * B], offsets[(t + 1) * B]
        modded[s:e] = np.mod(modded[s:e], rows[t])  # numpy integer mod is floor modulo
    plain = orc.emb_bag_fwd(W, "f64", row_offset, modded.astype(np.int32), offsets, B, D, "f64")
    assert np.array_equal(hashed, plain)
    with pytest.raises(ValueError):
        orc.emb_bag_fwd(W, "f64", row_offset, indices, offsets, B, D, "f64", hash_indices=False)


def test_emb_bag_rounding_is_single_rne():
    rng = np.random.default_rng(4)
    F, B, D = 2, 9, 8
    rows = [6, 6]
    row_offset, offsets, indices = make_problem(rng, F, B, rows, D, lengths=5)
    W = rng.normal(size=(12, D)).astype(np.float32)
    exact = orc.emb_bag_fwd(W, "f32", row_offset, indices, offsets, B, D, "f64")
    as_bf16 = orc.emb_bag_fwd(W, "f32", row_offset, indices, offsets, B, D, "bf16")
    as_f16 = orc.emb_bag_fwd(W, "f32", row_offset, indices, offsets, B, D, "f16")
    assert np.array_equal(as_f16.view(np.uint16), exact.astype(np.float16).view(np.uint16))
    flat = exact.reshape(-1)
    for x, o in zip(flat[:200], as_bf16.reshape(-1)[:200]):
        assert int(o) == nearest_bf16_bruteforce(float(x))


# ----------------------------------------------------------------------------------------
# dot interaction forward
# ----------------------------------------------------------------------------------------

def gram_reference(x0, emb):
    """[x0 | tril(V V^T, -1) row-major] with numpy's matmul and tril indices."""
    B, F, D = emb.shape
    Vm = np.concatenate([x0[:, None, :], emb], axis=1)  # [B][V][D]
    Z = Vm @ np.transpose(Vm, (0, 2, 1))
    i, j = np.tril_indices(F + 1, -1)  # row-major over the strict lower triangle
    return np.concatenate([x0, Z[:, i, j]], axis=1), Z


@pytest.mark.parametrize("F,D", [(1, 4), (8, 16), (26, 128), (5, 3)])
def test_dot_fwd_equals_masked_gram(F, D):
    rng = np.random.default_rng(5 + F)
    B = 6
    x0 = rng.normal(size=(B, D))
    emb = rng.normal(size=(B, F, D))
    V = F + 1
    P = V * (V - 1) // 2
    stride = D + P + 3
    out = orc.dot_interact_fwd(x0, emb, "f64", "f64", stride)
    ref, _ = gram_reference(x0, emb)
    np.testing.assert_allclose(out[:, :D + P], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out[:, :D], x0)
    assert np.all(out[:, D + P:] == 0) and not np.any(np.signbit(out[:, D + P:]))


def test_dot_fwd_two_vectors_is_one_dot_product():
    rng = np.random.default_rng(6)
    x0 = rng.normal(size=(4, 9)).astype(np.float32)
    emb = rng.normal(size=(4, 1, 9)).astype(np.float32)
    out = orc.dot_interact_fwd(x0, emb, "f32", "f64", 10)
    for b in range(4):
        assert out[b, 9] == pytest.approx(float(np.dot(x0[b].astype(np.float64), emb[b, 0].astype(np.float64))), rel=1e-15)


def test_dot_fwd_pair_sum_closed_form():
    rng = np.random.default_rng(7)
    B, F, D = 5, 26, 32
    x0 = rng.normal(size=(B, D))
    emb = rng.normal(size=(B, F, D))
    V = F + 1
    P = V * (V - 1) // 2
    out = orc.dot_interact_fwd(x0, emb, "f64", "f64", D + P)
    Vm = np.concatenate([x0[:, None, :], emb], axis=1)
    closed = (np.sum(Vm.sum(axis=1) ** 2, axis=1) - np.sum(Vm ** 2, axis=(1, 2))) / 2
    np.testing.assert_allclose(out[:, D:].sum(axis=1), closed, rtol=1e-10)


def test_dot_fwd_bf16_output_rounding():
    rng = np.random.default_rng(8)
    B, F, D = 3, 4, 16
    x0 = orc.round_from_f64(rng.normal(size=(B, D)), "bf16")
    emb = orc.round_from_f64(rng.normal(size=(B, F, D)), "bf16")
    exact = orc.dot_interact_fwd(x0, emb, "bf16", "f64", 26)
    got = orc.dot_interact_fwd(x0, emb, "bf16", "bf16", 26)
    for x, o in zip(exact.reshape(-1), got.reshape(-1)):
        assert int(o) == nearest_bf16_bruteforce(float(x))


# ----------------------------------------------------------------------------------------
# dot interaction backward
# ----------------------------------------------------------------------------------------

def loss_numpy(x0, emb, G):
    ref, _ = gram_reference(x0, emb)
    return float(np.sum(G[:, :ref.shape[1]] * ref))


@pytest.mark.parametrize("F,D", [(3, 4), (8, 16)])
def test_dot_bwd_central_differences_exact_for_quadratic(F, D):
    rng = np.random.default_rng(9)
    B = 2
    V = F + 1
    P = V * (V - 1) // 2
    x0 = rng.normal(size=(B, D))
    emb = rng.normal(size=(B, F, D))
    G = rng.normal(size=(B, D + P + 2))
    dx0, demb = orc.dot_interact_bwd(x0, emb, "f64", G, "f64", "f64")
    h = 0.25  # the loss is quadratic: central differences are exact for any step
    for arr, grad in ((x0, dx0), (emb, demb)):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = arr[ix]
            arr[ix] = old + h
            lp = loss_numpy(x0, emb, G)
            arr[ix] = old - h
            lm = loss_numpy(x0, emb, G)
            arr[ix] = old
            assert grad[ix] == pytest.approx((lp - lm) / (2 * h), rel=1e-9, abs=1e-9)


def test_dot_bwd_matches_symmetric_matrix_product_and_euler():
    rng = np.random.default_rng(10)
    B, F, D = 4, 26, 64
    V = F + 1
    P = V * (V - 1) // 2
    x0 = rng.normal(size=(B, D))
    emb = rng.normal(size=(B, F, D))
    G = rng.normal(size=(B, D + P))
    dx0, demb = orc.dot_interact_bwd(x0, emb, "f64", G, "f64", "f64")
    i, j = np.tril_indices(V, -1)
    Vm = np.concatenate([x0[:, None, :], emb], axis=1)
    for b in range(B):
        S = np.zeros((V, V))
        S[i, j] = G[b, D:]
        S = S + S.T
        dV = S @ Vm[b]
        np.testing.assert_allclose(dx0[b], G[b, :D] + dV[0], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(demb[b], dV[1:], rtol=1e-11, atol=1e-11)
        # Euler: sum_k <dV_k, V_k> = <G[:D], x0> + 2 <G_pairs, Z_pairs>
        lhs = np.dot(dx0[b], x0[b]) + np.sum(demb[b] * emb[b])
        Z = Vm[b] @ Vm[b].T
        rhs = np.dot(G[b, :D], x0[b]) + 2 * np.dot(G[b, D:], Z[i, j])
        assert lhs == pytest.approx(rhs, rel=1e-10)


def test_dot_bwd_ignores_padding_columns():
    rng = np.random.default_rng(11)
    B, F, D = 3, 4, 8
    P = (F + 1) * F // 2
    x0 = rng.normal(size=(B, D))
    emb = rng.normal(size=(B, F, D))
    G = rng.normal(size=(B, D + P + 5))
    G2 = G.copy()
    G2[:, D + P:] = 1e6
    a = orc.dot_interact_bwd(x0, emb, "f64", G, "f64", "f64")
    b = orc.dot_interact_bwd(x0, emb, "f64", G2, "f64", "f64")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------------------
# "cat" interaction (--interaction_op cat): the sample's vectors side by side
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("F,D,pad", [(1, 4, 0), (8, 16, 5), (26, 128, 0), (5, 3, 1)])
def test_cat_fwd_equals_numpy_stack_of_the_vectors(F, D, pad):
    """numpy's stack of [x0, emb[0], ..., emb[F-1]] along a new axis, flattened per sample
    (vector 0 = the bottom-MLP output, vector 1+t = table t), then zeros."""
    rng = np.random.default_rng(30 + F)
    B = 7
    x0 = rng.normal(size=(B, D))
    emb = rng.normal(size=(B, F, D))
    V = F + 1
    out = orc.cat_interact_fwd(x0, emb, "f64", "f64", V * D + pad)
    ref = np.stack([x0] + [emb[:, t, :] for t in range(F)], axis=1).reshape(B, V * D)
    assert np.array_equal(out[:, :V * D], ref)
    assert np.all(out[:, V * D:] == 0) and not np.any(np.signbit(out[:, V * D:]))


def test_cat_fwd_blocks_are_the_vectors_the_dot_interaction_multiplies():
    """The cat output's D-wide blocks, as a [V][D] matrix R, give numpy's Gram matrix
    R R^T whose strict lower triangle is the dot interaction's pair output (same vector
    order), and block 0 is the dot interaction's x0 copy."""
    rng = np.random.default_rng(31)
    B, F, D = 5, 6, 8
    x0 = rng.normal(size=(B, D))
    emb = rng.normal(size=(B, F, D))
    V = F + 1
    cat = orc.cat_interact_fwd(x0, emb, "f64", "f64", V * D)
    _, Z = gram_reference(x0, emb)
    R = cat.reshape(B, V, D)
    np.testing.assert_allclose(R @ np.transpose(R, (0, 2, 1)), Z, rtol=1e-13, atol=1e-13)
    assert np.array_equal(R[:, 0, :], x0)


def test_cat_fwd_bf16_is_an_exact_copy_and_f32_narrowing_rounds_once():
    rng = np.random.default_rng(32)
    B, F, D = 4, 3, 16
    x0 = orc.round_from_f64(rng.normal(size=(B, D)), "bf16")
    emb = orc.round_from_f64(rng.normal(size=(B, F, D)), "bf16")
    out = orc.cat_interact_fwd(x0, emb, "bf16", "bf16", (F + 1) * D + 8)
    assert np.array_equal(out[:, :D], x0)
    assert np.array_equal(out[:, D:(F + 1) * D].reshape(B, F, D), emb)
    assert np.all(out[:, (F + 1) * D:] == 0)
    # fp32 in, bf16 out: each element rounded once, to the nearest bf16 (exhaustive search)
    x32 = rng.normal(size=(B, D)).astype(np.float32)
    e32 = rng.normal(size=(B, F, D)).astype(np.float32)
    o16 = orc.cat_interact_fwd(x32, e32, "f32", "bf16", (F + 1) * D)
    for x, o in zip(np.concatenate([x32, e32.reshape(B, -1)], 1).reshape(-1)[:300], o16.reshape(-1)[:300]):
        assert int(o) == nearest_bf16_bruteforce(float(x))


def cat_loss_numpy(x0, emb, G):
    """sum G * [x0 | emb flattened] (numpy; linear in the inputs)."""
    B, F, D = emb.shape
    return float(np.sum(G[:, :D] * x0) + np.sum(G[:, D:(F + 1) * D] * emb.reshape(B, F * D)))


def test_cat_bwd_central_differences_and_adjoint_identity():
    """The loss sum G * out is linear in (x0, emb): central differences are exact, and the
    backward is the adjoint of the forward, <G, cat(x0, emb)> = <dx0, x0> + <demb, emb>."""
    rng = np.random.default_rng(33)
    B, F, D = 3, 4, 5
    x0 = rng.normal(size=(B, D))
    emb = rng.normal(size=(B, F, D))
    G = rng.normal(size=(B, (F + 1) * D + 3))
    dx0, demb = orc.cat_interact_bwd(G, "f64", F, D, "f64")
    h = 0.5
    for arr, grad in ((x0, dx0), (emb, demb)):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = arr[ix]
            arr[ix] = old + h
            lp = cat_loss_numpy(x0, emb, G)
            arr[ix] = old - h
            lm = cat_loss_numpy(x0, emb, G)
            arr[ix] = old
            assert grad[ix] == pytest.approx((lp - lm) / (2 * h), rel=1e-12, abs=1e-12)
    out = orc.cat_interact_fwd(x0, emb, "f64", "f64", G.shape[1])
    lhs = float(np.sum(G * out))
    rhs = float(np.sum(dx0 * x0) + np.sum(demb * emb))
    assert lhs == pytest.approx(rhs, rel=1e-12)


def test_cat_bwd_of_the_forward_output_returns_the_inputs_and_ignores_padding():
    """Special case: with G = the forward's own output the gradient blocks are the inputs
    themselves (bit for bit); padding columns of G do not matter."""
    rng = np.random.default_rng(34)
    B, F, D = 6, 7, 8
    x0 = orc.round_from_f64(rng.normal(size=(B, D)), "bf16")
    emb = orc.round_from_f64(rng.normal(size=(B, F, D)), "bf16")
    S = (F + 1) * D + 8
    out = orc.cat_interact_fwd(x0, emb, "bf16", "bf16", S)
    out[:, (F + 1) * D:] = 0x7F00  # large values in the padding
    dx0, demb = orc.cat_interact_bwd(out, "bf16", F, D, "bf16")
    assert np.array_equal(dx0, x0) and np.array_equal(demb, emb)


# ----------------------------------------------------------------------------------------
# sort, segments, reduce + SGD
# ----------------------------------------------------------------------------------------

def keys_and_bags(row_offset, offsets, indices, B, hash_indices=False):
    F = row_offset.size - 1
    keys, bags = [], []
    for t in range(F):
        n = int(row_offset[t + 1] - row_offset[t])
        for b in range(B):
            g = t * B + b
            for k in range(offsets[g], offsets[g + 1]):
                r = int(indices[k])
                if hash_indices:
                    r %= n
                keys.append(int(row_offset[t]) + r)
                bags.append(g)
    return np.array(keys, np.int64), np.array(bags, np.int64)


@pytest.mark.parametrize("hash_indices", [False, True])
def test_grad_sort_matches_numpy_stable_argsort(hash_indices):
    rng = np.random.default_rng(12)
    F, B = 4, 50
    rows = [30, 3, 100, 17]
    row_offset, offsets, indices = make_problem(rng, F, B, rows, 1, lengths=4, hash_range=hash_indices)
    s = orc.grad_sort(row_offset, indices, offsets, B, hash_indices=hash_indices)
    keys, bags = keys_and_bags(row_offset, offsets, indices, B, hash_indices)
    order = np.argsort(keys, kind="stable")
    assert np.array_equal(s["sorted_rows"], keys[order])
    assert np.array_equal(s["bag_ids"], bags[order])
    uniq, first = np.unique(keys[order], return_index=True)
    assert np.array_equal(s["unique_rows"], uniq)
    assert np.array_equal(s["seg_offsets"], np.append(first, keys.size))
    assert s["num_unique"] == uniq.size


def test_grad_sort_counting_sort_on_tiny_key_range():
    rng = np.random.default_rng(13)
    F, B = 2, 40
    rows = [3, 2]
    row_offset, offsets, indices = make_problem(rng, F, B, rows, 1, lengths=3)
    s = orc.grad_sort(row_offset, indices, offsets, B)
    keys, bags = keys_and_bags(row_offset, offsets, indices, B)
    buckets = [[] for _ in range(5)]
    for k, g in zip(keys, bags):  # counting sort: append in lookup order
        buckets[k].append((k, g))
    flat = [x for bk in buckets for x in bk]
    assert [int(v) for v in s["sorted_rows"]] == [k for k, _ in flat]
    assert [int(v) for v in s["bag_ids"]] == [g for _, g in flat]


def dense_sgd(W, row_offset, offsets, indices, B, demb, lr, hash_indices=False):
    """Brute force: accumulate the full dense gradient dW in lookup order, then SGD on
    every row of the table."""
    F = row_offset.size - 1
    dW = np.zeros_like(W, dtype=np.float64)
    keys, bags = keys_and_bags(row_offset, offsets, indices, B, hash_indices)
    for k, g in zip(keys, bags):
        t, b = divmod(int(g), B)
        dW[k] += demb[b, t]
    return W - np.float64(np.float32(lr)) * dW


@pytest.mark.parametrize("lengths", ["one", 5])
def test_grad_update_equals_dense_sgd(lengths):
    rng = np.random.default_rng(14)
    F, B, D = 3, 20, 6
    rows = [9, 30, 4]
    row_offset, offsets, indices = make_problem(rng, F, B, rows, D, lengths=lengths)
    W = rng.normal(0, 0.01, size=(sum(rows), D))
    demb = rng.normal(size=(B, F, D))
    new = orc.grad_reduce_update(W, "f64", row_offset, indices, offsets, B, demb, "f64", 0.01)
    ref = dense_sgd(W, row_offset, offsets, indices, B, demb, 0.01)
    assert np.array_equal(new, ref)  # same summation order per row: bit-exact in float64


def test_grad_update_invariants():
    rng = np.random.default_rng(15)
    F, B, D = 4, 64, 8
    rows = [100, 100, 5, 40]
    row_offset, offsets, indices = make_problem(rng, F, B, rows, D, lengths=3)
    W32 = rng.normal(0, 0.01, size=(sum(rows), D)).astype(np.float32)
    demb = rng.normal(size=(B, F, D)).astype(np.float32)
    # lr = 0: bitwise unchanged
    same = orc.grad_reduce_update(W32, "f32", row_offset, indices, offsets, B, demb, "f32", 0.0)
    assert np.array_equal(same.view(np.uint32), W32.view(np.uint32))
    # untouched rows bitwise unchanged; touched rows are exactly the looked-up rows
    new = orc.grad_reduce_update(W32, "f32", row_offset, indices, offsets, B, demb, "f32", 0.01)
    keys, bags = keys_and_bags(row_offset, offsets, indices, B)
    touched = np.zeros(W32.shape[0], bool)
    touched[keys] = True
    assert np.array_equal(new[~touched].view(np.uint32), W32[~touched].view(np.uint32))
    # column-sum conservation (float64 tables): sum(W_new - W_old) = -lr * sum_k demb[bag_k]
    W64 = W32.astype(np.float64)
    d64 = demb.astype(np.float64)
    new64 = orc.grad_reduce_update(W64, "f64", row_offset, indices, offsets, B, d64, "f64", 0.01)
    tot = np.zeros(D)
    for g in bags:
        t, b = divmod(int(g), B)
        tot += d64[b, t]
    np.testing.assert_allclose((new64 - W64).sum(axis=0), -np.float64(np.float32(0.01)) * tot, rtol=1e-9, atol=1e-12)


def test_grad_update_single_repeated_row_is_column_sum():
    F, B, D = 1, 37, 4
    row_offset = np.array([0, 10], np.int64)
    offsets = np.arange(B + 1, dtype=np.int32)
    indices = np.full(B, 6, np.int32)
    rng = np.random.default_rng(16)
    W = rng.normal(size=(10, D))
    demb = rng.normal(size=(B, F, D))
    s = orc.grad_sort(row_offset, indices, offsets, B)
    assert s["num_unique"] == 1 and list(s["seg_offsets"]) == [0, B]
    new = orc.grad_reduce_update(W, "f64", row_offset, indices, offsets, B, demb, "f64", 0.5)
    expect = W[6] - np.float64(np.float32(0.5)) * np.cumsum(demb[:, 0, :], axis=0)[-1]
    np.testing.assert_allclose(new[6], expect, rtol=1e-14)
    assert np.array_equal(np.delete(new, 6, axis=0), np.delete(W, 6, axis=0))


def test_bad_offsets_rejected():
    row_offset = np.array([0, 4], np.int64)
    offsets = np.array([0, 2, 1], np.int32)
    with pytest.raises(ValueError):
        orc.emb_bag_fwd(np.zeros((4, 2)), "f64", row_offset, np.zeros(2, np.int32), offsets, 2, 2, "f64")


def test_openmp_build_gives_the_plain_builds_bits():
    """The OpenMP build of the oracle (used only to time the CPU baseline on all host
    threads) splits independent bags / samples over threads and must give the plain build's
    bits."""
    import os
    from oracle import build as obuild
    if not os.path.exists(obuild.LIB_OMP):
        obuild.build()
    rng = np.random.default_rng(11)
    F, B, D = 5, 37, 24
    rows = np.array([7, 30, 1, 12, 50])
    ro = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    W = rng.standard_normal((int(ro[-1]), D)).astype(np.float32)
    lens = rng.integers(0, 4, F * B)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t_of = np.repeat(np.arange(F).repeat(B), lens)
    idx = (rng.integers(0, 1 << 20, off[-1]) % rows[t_of]).astype(np.int32)
    x0 = rng.standard_normal((B, D)).astype(np.float32)
    S = D + (F + 1) * F // 2
    G = rng.standard_normal((B, S)).astype(np.float32)

    def chain():
        emb = orc.emb_bag_fwd(W, "f32", ro, idx, off, B, D, "f32")
        out = orc.dot_interact_fwd(x0, emb, "f32", "f32", S)
        dx0, demb = orc.dot_interact_bwd(x0, emb, "f32", G, "f32", "f32")
        return [a.copy() for a in (emb, out, dx0, demb)]

    plain = chain()
    prev = orc.use_library(obuild.LIB_OMP)
    try:
        threaded = chain()
    finally:
        orc.restore_library(prev)
    for a, b in zip(plain, threaded):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ----------------------------------------------------------------------------------------
# dense layers, logistic loss, dense SGD (page "DLRM For PyTorch", §Model architecture:
# bottom MLP = linear layers with ReLU; top MLP ending in one logit; --bottom_mlp_sizes,
# --top_mlp_sizes)
# ----------------------------------------------------------------------------------------

def _exact_grid(rng, shape, lo=-8, hi=9, scale=0.125):
    """Small multiples of 1/8: exact in bf16, and every product and short sum of them is
    exact in binary32 and binary64."""
    return rng.integers(lo, hi, size=shape).astype(np.float64) * scale


@pytest.mark.parametrize("relu", [False, True])
def test_linear_fwd_matches_float64_matmul_on_exact_values(relu):
    """Library routine: float64 matmul.  On values whose sums are exact, the oracle's bf16
    output must be torch's bf16 rounding of numpy's result, bit for bit; with random float64
    inputs it must agree with numpy to float64 rounding."""
    rng = np.random.default_rng(5)
    M, K, N = 9, 12, 7
    x, w = _exact_grid(rng, (M, K)), _exact_grid(rng, (N, K))
    b = _exact_grid(rng, (N,)).astype(np.float32)
    ref = x @ w.T + b
    if relu:
        ref = np.maximum(ref, 0.0)
    xb, wb = f32_to_bf16_bits_torch(x), f32_to_bf16_bits_torch(w)
    got = orc.linear_fwd(xb, "bf16", wb, "bf16", b, relu, "bf16")
    assert np.array_equal(got, f32_to_bf16_bits_torch(ref))
    xr, wr = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    ref = xr @ wr.T + b
    if relu:
        ref = np.maximum(ref, 0.0)
    got = orc.linear_fwd(xr, "f64", wr, "f64", b, relu, "f64")
    assert np.max(np.abs(got - ref)) < 1e-12


def test_linear_fwd_respects_row_strides():
    """Special case: a layer over the first K columns of a wider row equals the layer over
    the sliced matrix; the output's extra columns are not written."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 16))
    w = rng.standard_normal((3, 13))
    got = orc.linear_fwd(x, "f64", w, "f64", None, False, "f64", K=13, ldy=8)
    ref = orc.linear_fwd(np.ascontiguousarray(x[:, :13]), "f64", w, "f64", None, False, "f64")
    assert np.array_equal(got[:, :3], ref)
    assert np.all(np.isnan(got[:, 3:]))


def test_linear_bwd_central_differences_exact():
    """L = sum(G * (x W^T + b)) is linear in each of x, W, b, so central differences give the
    exact partial derivatives (up to float64 rounding): they must equal dx, dW, db of the
    backward with dz = G."""
    rng = np.random.default_rng(7)
    M, K, N = 5, 4, 3
    x, w = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    b = rng.standard_normal(N).astype(np.float32).astype(np.float64)
    G = rng.standard_normal((M, N))

    def L(x_, w_, b_):
        y = orc.linear_fwd(x_, "f64", w_, "f64", None, False, "f64")
        return float(np.sum(G * (y + b_)))

    dx, dw, db = orc.linear_bwd(x, "f64", w, "f64", G, "f64", dx_dtype="f64", wgrad_dtype="f64")
    h = 0.5
    for (arr, grad) in ((x, dx), (w, dw)):
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = (p, w, b) if arr is x else (x, p, b)
            args_m = (m, w, b) if arr is x else (x, m, b)
            fd = (L(*args_p) - L(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-10 * max(1.0, abs(fd))
    for n in range(N):
        p, m = b.copy(), b.copy()
        p[n] += h
        m[n] -= h
        assert abs((L(x, w, p) - L(x, w, m)) / (2 * h) - db[n]) < 1e-10


def test_linear_bwd_mask_is_the_relu_derivative():
    """With the ReLU mask, dx is the derivative of sum(G * (relu(x) W^T)) w.r.t. x: checked by
    central differences at points away from the kink (x = 0 entries give 0)."""
    rng = np.random.default_rng(8)
    M, K, N = 4, 6, 5
    x = rng.standard_normal((M, K))
    x[np.abs(x) < 0.2] = 0.5
    x[0, 0] = 0.0
    w, G = rng.standard_normal((N, K)), rng.standard_normal((M, N))
    dx, _, _ = orc.linear_bwd(x, "f64", w, "f64", G, "f64", dx_dtype="f64", relu_mask=True,
                              wgrad_dtype="f64")

    def L(x_):
        return float(np.sum(G * (np.maximum(x_, 0.0) @ w.T)))

    h = 0.05
    for idx in np.ndindex(x.shape):
        if x[idx] == 0.0:
            assert dx[idx] == 0.0
            continue
        p, m = x.copy(), x.copy()
        p[idx] += h
        m[idx] -= h
        assert abs((L(p) - L(m)) / (2 * h) - dx[idx]) < 1e-10


def test_linear_bwd_transposition_identity():
    """<dx, x> = <dW, W> = sum(dz * (x W^T)): both gradients contract the same bilinear form."""
    rng = np.random.default_rng(9)
    M, K, N = 7, 5, 6
    x, w, dz = rng.standard_normal((M, K)), rng.standard_normal((N, K)), rng.standard_normal((M, N))
    dx, dw, db = orc.linear_bwd(x, "f64", w, "f64", dz, "f64", dx_dtype="f64", wgrad_dtype="f64")
    ref = float(np.sum(dz * (x @ w.T)))
    assert abs(np.sum(dx * x) - ref) < 1e-10
    assert abs(np.sum(dw * w) - ref) < 1e-10
    assert np.max(np.abs(db - dz.sum(axis=0))) < 1e-12


def test_bce_closed_forms():
    """z = 0: loss log 2, dz = (1/2 - y)/M.  Label symmetry loss(z, y) = loss(-z, 1 - y).
    Saturation: z = -1000, y = 1 costs 1000 and z = 1000, y = 1 costs 0, with no overflow."""
    y = np.array([0, 1, 1, 0], np.float32)
    loss, dz = orc.bce_logits(np.zeros(4), "f64", y, "f64")
    assert abs(loss - np.log(2.0)) < 1e-15
    assert np.array_equal(dz, (0.5 - y) / 4)
    rng = np.random.default_rng(10)
    z = rng.standard_normal(64) * 5
    lab = (rng.random(64) < 0.3).astype(np.float32)
    l1, _ = orc.bce_logits(z, "f64", lab, "f64")
    l2, _ = orc.bce_logits(-z, "f64", 1 - lab, "f64")
    assert abs(l1 - l2) < 1e-14
    l3, d3 = orc.bce_logits(np.array([-1000.0, 1000.0]), "f64", np.array([1, 1], np.float32), "f64")
    assert abs(l3 - 500.0) < 1e-12
    assert np.array_equal(d3, np.array([-0.5, 0.0]))
    # -log of the predicted probability of the true label, term by term
    p = 1 / (1 + np.exp(-z))
    ref = -np.mean(np.where(lab == 1, np.log(p), np.log1p(-p)))
    assert abs(l1 - ref) < 1e-12


def test_bce_gradient_central_differences():
    rng = np.random.default_rng(12)
    M = 16
    z = rng.standard_normal(M) * 3
    lab = (rng.random(M) < 0.5).astype(np.float32)
    _, dz = orc.bce_logits(z, "f64", lab, "f64")
    h = 1e-5
    for m in range(M):
        p, q = z.copy(), z.copy()
        p[m] += h
        q[m] -= h
        fd = (orc.bce_logits(p, "f64", lab, "f64")[0] - orc.bce_logits(q, "f64", lab, "f64")[0]) / (2 * h)
        assert abs(fd - dz[m]) < 1e-9


def test_sgd_dense_special_cases():
    """lr = 0 keeps the master bits; an exact step; the 16-bit copy is torch's rounding of the
    new master."""
    rng = np.random.default_rng(13)
    m = rng.standard_normal(257).astype(np.float32)
    g = rng.standard_normal(257).astype(np.float32)
    new, copy = orc.sgd_dense(m, g, 0.0, "bf16")
    assert np.array_equal(new.view(np.uint32), m.view(np.uint32))
    assert np.array_equal(copy, f32_to_bf16_bits_torch(m))
    new, _ = orc.sgd_dense(np.array([1.0, -3.0], np.float32), np.array([2.0, 4.0], np.float32), 0.25)
    assert np.array_equal(new, np.array([0.5, -4.0], np.float32))
    new, copy = orc.sgd_dense(m, g, 0.01, "bf16")
    ref = (m.astype(np.float64) - np.float64(np.float32(0.01)) * g.astype(np.float64)).astype(np.float32)
    assert np.array_equal(new.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(copy, f32_to_bf16_bits_torch(ref))


def test_mlp_chain_gradient_central_differences():
    """A two-layer ReLU MLP, one logit and the logistic loss, all in float64: the backward
    chain (loss gradient -> logit layer -> masked hidden layer) must match central differences
    of the loss w.r.t. the first layer's weights and the dense input."""
    rng = np.random.default_rng(14)
    M, K, H = 6, 5, 4
    x = rng.standard_normal((M, K))
    w1, b1 = rng.standard_normal((H, K)), rng.standard_normal(H).astype(np.float32)
    w2, b2 = rng.standard_normal((1, H)), rng.standard_normal(1).astype(np.float32)
    lab = (rng.random(M) < 0.5).astype(np.float32)

    def loss(x_, w1_):
        h1 = orc.linear_fwd(x_, "f64", w1_, "f64", b1, True, "f64")
        z = orc.linear_fwd(h1, "f64", w2, "f64", b2, False, "f64")
        return orc.bce_logits(z, "f64", lab, "f64")[0]

    h1 = orc.linear_fwd(x, "f64", w1, "f64", b1, True, "f64")
    z = orc.linear_fwd(h1, "f64", w2, "f64", b2, False, "f64")
    _, dz = orc.bce_logits(z, "f64", lab, "f64")
    dh1, _, _ = orc.linear_bwd(h1, "f64", w2, "f64", dz.reshape(M, 1), "f64", dx_dtype="f64",
                               relu_mask=True, wgrad_dtype="f64")
    dx, dw1, _ = orc.linear_bwd(x, "f64", w1, "f64", dh1, "f64", dx_dtype="f64", wgrad_dtype="f64")
    h = 1e-6
    for arr, grad, which in ((w1, dw1, 1), (x, dx, 0)):
        for idx in list(np.ndindex(arr.shape))[:12]:
            p, q = arr.copy(), arr.copy()
            p[idx] += h
            q[idx] -= h
            fd = (loss(p, w1) - loss(q, w1)) / (2 * h) if which == 0 else \
                (loss(x, p) - loss(x, q)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7


def test_relu_bwd_is_the_relu_derivative():
    """dz = dy where y > 0, else 0 (y = 0 at the kink, negative zero and NaN give 0): the
    derivative of the ReLU, written out element by element."""
    rng = np.random.default_rng(15)
    dy = rng.standard_normal((3, 5))
    y = np.maximum(rng.standard_normal((3, 5)), 0.0)
    y[0, 0], y[0, 1], y[0, 2] = 0.0, -0.0, np.nan
    dz = orc.relu_bwd(dy, y, "f64")
    for idx in np.ndindex(y.shape):
        assert dz[idx] == (dy[idx] if y[idx] > 0 else 0.0)
    assert np.count_nonzero(dz) == np.count_nonzero(y > 0)
