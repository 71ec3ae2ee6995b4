"""The C-ABI library loads, exports what include/embcore.h declares, and rejects bad
arguments on the host before anything reaches a GPU (no compute call is made here)."""
import ctypes

import pytest

from embedding_lookup_feature_amd import embcore as ec

INVALID, UNSUPPORTED, WORKSPACE = ec.EL_ERR_INVALID_ARG, ec.EL_ERR_UNSUPPORTED, ec.EL_ERR_WORKSPACE

# Fake but aligned device addresses: every call below fails validation before any use.
A = 0x7F0000000000


def tables(F=26, D=128, rows=100_000, dtype=ec.EL_F32, base=A, row_offset=A + 0x1000, max_rows=0):
    return ec.ElTables(base, row_offset, F * rows, F, D, dtype, max_rows)


def bags(F=26, B=65536, nnz=None, indices=A + 0x2000, offsets=A + 0x3000):
    return ec.ElBags(indices, offsets, B, F * B if nnz is None else nnz)


def ref(x):
    return ctypes.byref(x)


def test_library_loads_and_exports_every_declared_function():
    L = ec.lib()
    names = ec.header_functions()
    assert set(names) == {"emb_bag_fwd", "dot_interact_fwd", "emb_dot_fwd", "dot_interact_bwd", "emb_dot_bwd",
                          "emb_grad_workspace_bytes", "emb_grad_reduce_update",
                          "emb_grad_reduce_update_noalloc", "emb_grad_prepare",
                          "cat_interact_fwd", "cat_interact_bwd", "emb_cat_fwd", "el_hbm_calib",
                          "emb_grad_apply", "emb_grad_sort",
                          "el_validate_bags", "el_last_error", "el_version", "el_linear_fwd",
                          "el_linear_bwd_workspace_bytes", "el_linear_bwd", "el_relu_bwd",
                          "el_bce_workspace_bytes", "el_bce_logits", "el_sgd_dense"}
    for n in names:
        assert hasattr(L, n), n
    assert ec.el_version() == 200


def test_workspace_bytes_is_host_pure_and_scales():
    L = ec.lib()
    small = L.emb_grad_workspace_bytes(ref(tables()), ref(bags(B=1024)))
    big = L.emb_grad_workspace_bytes(ref(tables()), ref(bags()))
    assert 0 < small < big
    # 4 key/value arrays + 2 flag arrays of nnz words, plus histograms and partials
    nnz = 26 * 65536
    assert big >= 6 * 4 * nnz
    assert L.emb_grad_workspace_bytes(ref(tables()), ref(bags(B=0, nnz=0))) == 0
    assert L.emb_grad_workspace_bytes(None, ref(bags())) == 0
    # a declared largest table: the sort works on fewer bits (17 instead of 22 here: 2
    # passes of 9-bit digits instead of 3 of 8, so a larger digit histogram, still far
    # below the key arrays); beyond the total it is refused
    declared = L.emb_grad_workspace_bytes(ref(tables(max_rows=100_000)), ref(bags()))
    assert 6 * 4 * nnz <= declared <= big + 4 * (26 + nnz // 4096 + 1) * 512 * 2
    assert L.emb_grad_workspace_bytes(ref(tables(max_rows=26 * 100_000 + 1)), ref(bags())) == 0
    assert L.emb_grad_workspace_bytes(ref(tables(max_rows=-1)), ref(bags())) == 0


@pytest.mark.parametrize("tab,bg,flags,out,odt,status", [
    (None, bags(), 0, A, ec.EL_BF16, INVALID),
    (tables(F=0), bags(), 0, A, ec.EL_BF16, INVALID),
    (tables(D=3), bags(), 0, A, ec.EL_BF16, UNSUPPORTED),      # 12-byte rows
    (tables(base=A + 8), bags(), 0, A, ec.EL_BF16, INVALID),   # misaligned table
    (tables(), bags(nnz=1 << 31), 0, A, ec.EL_BF16, INVALID),
    (tables(), bags(B=-1), 0, A, ec.EL_BF16, INVALID),
    (tables(), bags(), 2, A, ec.EL_BF16, INVALID),             # unknown flag
    (tables(), bags(), 0, A + 4, ec.EL_BF16, INVALID),         # misaligned output
    (tables(), bags(), 0, 0, ec.EL_BF16, INVALID),             # null output
    (tables(), bags(), 0, A, 7, INVALID),                      # unknown dtype
    (tables(dtype=9), bags(), 0, A, ec.EL_BF16, INVALID),
    (tables(), bags(offsets=0), 0, A, ec.EL_BF16, INVALID),
])
def test_emb_bag_fwd_rejects(tab, bg, flags, out, odt, status):
    L = ec.lib()
    rc = L.emb_bag_fwd(ref(tab) if tab is not None else None, ref(bg), flags, out, odt, None)
    assert rc == status
    assert "emb_bag_fwd" in ec.el_last_error()


def test_emb_dot_fwd_rejects():
    L = ec.lib()
    T, Bg = ref(tables()), ref(bags())
    assert L.emb_dot_fwd(T, Bg, 0, A, ec.EL_BF16, A, A, 478, None) == INVALID      # out_stride < D + P
    assert L.emb_dot_fwd(T, Bg, 4, A, ec.EL_BF16, A, A, 480, None) == INVALID      # unknown flag
    assert L.emb_dot_fwd(T, Bg, 0, 0, ec.EL_BF16, A, A, 480, None) == INVALID      # null x0
    assert L.emb_dot_fwd(T, Bg, 0, A, ec.EL_BF16, A + 8, A, 480, None) == INVALID  # misaligned emb_out
    assert L.emb_dot_fwd(T, Bg, 0, A, ec.EL_BF16, A, 0, 480, None) == INVALID      # null out
    assert L.emb_dot_fwd(T, Bg, 0, A, 6, A, A, 480, None) == INVALID               # unknown dtype
    assert L.emb_dot_fwd(None, Bg, 0, A, ec.EL_BF16, A, A, 480, None) == INVALID
    assert "emb_dot_fwd" in ec.el_last_error()
    # B == 0: valid, nothing enqueued
    assert L.emb_dot_fwd(T, ref(bags(B=0, nnz=0)), 0, A, ec.EL_BF16, None, A, 480, None) == ec.EL_OK


def test_emb_dot_fwd_unsupported_fused_shapes_say_why():
    """Without emb_out, shapes outside the fused kernel's classes are refused on the host with
    their own error text (not a stale one from an earlier call)."""
    L = ec.lib()
    assert L.emb_bag_fwd(None, ref(bags()), 0, A, ec.EL_BF16, None) == INVALID
    assert "emb_bag_fwd" in ec.el_last_error()
    # 65 vectors of 16: a 2096-element bf16 output row (4192 bytes) exceeds the fused kernel's
    # output-row classes
    rc = L.emb_dot_fwd(ref(tables(F=64, D=16)), ref(bags(F=64)), 0, A, ec.EL_BF16, None, A, 2096, None)
    assert rc == UNSUPPORTED
    assert "emb_dot_fwd" in ec.el_last_error() and "4096 bytes" in ec.el_last_error()
    # 64 tables of 256: more row chunks per sample than the fused kernel holds
    assert L.emb_bag_fwd(None, ref(bags()), 0, A, ec.EL_BF16, None) == INVALID
    rc = L.emb_dot_fwd(ref(tables(F=64, D=256)), ref(bags(F=64)), 0, A, ec.EL_BF16, None, A, 2336, None)
    assert rc == UNSUPPORTED
    assert "emb_dot_fwd" in ec.el_last_error()
    # fp32 activations without emb_out
    rc = L.emb_dot_fwd(ref(tables()), ref(bags()), 0, A, ec.EL_F32, None, A, 480, None)
    assert rc == UNSUPPORTED and "emb_dot_fwd" in ec.el_last_error()


def test_emb_dot_bwd_rejects():
    L = ec.lib()
    T, Bg = ref(tables()), ref(bags())
    bf = ec.EL_BF16
    assert L.emb_dot_bwd(T, Bg, 0, A, bf, A, 478, A, A, bf, None) == INVALID      # out_stride < D + P
    assert L.emb_dot_bwd(T, Bg, 4, A, bf, A, 480, A, A, bf, None) == INVALID      # unknown flag
    assert L.emb_dot_bwd(T, Bg, 0, 0, bf, A, 480, A, A, bf, None) == INVALID      # null x0
    assert L.emb_dot_bwd(T, Bg, 0, A, bf, A + 8, 480, A, A, bf, None) == INVALID  # misaligned dout
    assert L.emb_dot_bwd(T, Bg, 0, A, bf, A, 480, 0, A, bf, None) == INVALID      # null dx0
    assert L.emb_dot_bwd(T, Bg, 0, A, bf, A, 480, A, 0, bf, None) == INVALID      # null demb
    assert L.emb_dot_bwd(T, Bg, 0, A, bf, A, 480, A, A, 6, None) == INVALID       # unknown dtype
    assert L.emb_dot_bwd(None, Bg, 0, A, bf, A, 480, A, A, bf, None) == INVALID
    assert "emb_dot_bwd" in ec.el_last_error()
    # shapes outside the fused kernel: refused on the host, nothing enqueued
    assert L.emb_dot_bwd(ref(tables(F=40)), ref(bags(F=40)), 0, A, bf, A, 1000, A, A, bf, None) == UNSUPPORTED
    assert L.emb_dot_bwd(ref(tables(D=16)), Bg, 0, A, bf, A, 376, A, A, bf, None) == UNSUPPORTED
    assert L.emb_dot_bwd(T, Bg, 0, A, ec.EL_F32, A, 480, A, A, ec.EL_F32, None) == UNSUPPORTED
    assert "emb_dot_bwd" in ec.el_last_error()
    # B == 0: valid, nothing enqueued
    assert L.emb_dot_bwd(T, ref(bags(B=0, nnz=0)), 0, A, bf, A, 480, A, A, bf, None) == ec.EL_OK


def test_dot_interact_rejects():
    L = ec.lib()
    # out_stride below D + P
    assert L.dot_interact_fwd(A, A, ec.EL_BF16, 8, 26, 128, A, ec.EL_BF16, 478, None) == INVALID
    assert L.dot_interact_fwd(A, A, ec.EL_BF16, 8, 0, 128, A, ec.EL_BF16, 480, None) == INVALID
    assert L.dot_interact_fwd(A + 2, A, ec.EL_BF16, 8, 26, 128, A, ec.EL_BF16, 480, None) == INVALID
    assert L.dot_interact_fwd(A, A, 5, 8, 26, 128, A, ec.EL_BF16, 480, None) == INVALID
    assert L.dot_interact_fwd(A, A, ec.EL_BF16, -1, 26, 128, A, ec.EL_BF16, 480, None) == INVALID
    # B == 0 is a valid no-op that enqueues nothing
    assert L.dot_interact_fwd(A, A, ec.EL_BF16, 0, 26, 128, A, ec.EL_BF16, 480, None) == ec.EL_OK
    assert L.dot_interact_bwd(A, A, ec.EL_BF16, 8, 26, 128, A, ec.EL_BF16, 400, A, A, ec.EL_BF16, None) == INVALID
    assert L.dot_interact_bwd(A, A, ec.EL_BF16, 8, 26, 128, A, ec.EL_BF16, 480, 0, A, ec.EL_BF16, None) == INVALID
    assert "dot_interact_bwd" in ec.el_last_error()


def test_cat_calls_reject_on_the_host():
    L = ec.lib()
    bf = ec.EL_BF16
    # out_stride below (F+1) * D
    assert L.cat_interact_fwd(A, A, bf, 8, 26, 128, A, bf, 27 * 128 - 1, None) == INVALID
    assert L.cat_interact_fwd(A, A, bf, 8, 0, 128, A, bf, 27 * 128, None) == INVALID
    assert L.cat_interact_fwd(A + 2, A, bf, 8, 26, 128, A, bf, 27 * 128, None) == INVALID
    assert L.cat_interact_fwd(A, A, 5, 8, 26, 128, A, bf, 27 * 128, None) == INVALID
    assert L.cat_interact_fwd(A, A, bf, -1, 26, 128, A, bf, 27 * 128, None) == INVALID
    assert "cat_interact_fwd" in ec.el_last_error()
    assert L.cat_interact_fwd(A, A, bf, 0, 26, 128, A, bf, 27 * 128, None) == ec.EL_OK
    assert L.cat_interact_bwd(A, bf, 8, 26, 128, 27 * 128 - 8, A, A, bf, None) == INVALID
    assert L.cat_interact_bwd(A, bf, 8, 26, 128, 27 * 128, 0, A, bf, None) == INVALID
    assert L.cat_interact_bwd(A, bf, 8, 26, 128, 27 * 128, A, A + 4, bf, None) == INVALID
    assert "cat_interact_bwd" in ec.el_last_error()
    T, Bg = ref(tables()), ref(bags())
    assert L.emb_cat_fwd(T, Bg, 0, A, bf, A, 27 * 128 - 1, None) == INVALID
    assert L.emb_cat_fwd(T, Bg, 2, A, bf, A, 27 * 128, None) == INVALID
    assert L.emb_cat_fwd(T, Bg, 0, 0, bf, A, 27 * 128, None) == INVALID
    assert L.emb_cat_fwd(None, Bg, 0, A, bf, A, 27 * 128, None) == INVALID
    # a row stride that is not a multiple of 16 bytes: refused before anything is enqueued
    assert L.emb_cat_fwd(T, Bg, 0, A, bf, A, 27 * 128 + 3, None) == UNSUPPORTED
    assert "emb_cat_fwd" in ec.el_last_error()
    assert L.emb_cat_fwd(T, ref(bags(B=0, nnz=0)), 0, A, bf, A, 27 * 128, None) == ec.EL_OK


def test_hbm_calib_rejects_on_the_host():
    L = ec.lib()
    assert L.el_hbm_calib(9, A, A, 1 << 20, None, 0, 0, None) == INVALID
    assert L.el_hbm_calib(ec.EL_CALIB_COPY, A, A, 100, None, 0, 0, None) == INVALID      # not a multiple of 64
    assert L.el_hbm_calib(ec.EL_CALIB_COPY, 0, A, 1 << 20, None, 0, 0, None) == INVALID  # null src
    assert L.el_hbm_calib(ec.EL_CALIB_READ, A, A + 8, 1 << 20, None, 0, 0, None) == INVALID
    assert L.el_hbm_calib(ec.EL_CALIB_GATHER, A, A, 0, None, 10, 256, None) == INVALID     # null idx
    assert L.el_hbm_calib(ec.EL_CALIB_GATHER, A, A, 0, A, 10, 24, None) == INVALID         # row size
    assert L.el_hbm_calib(ec.EL_CALIB_GATHER, A, A, 0, A, 10, 2048, None) == INVALID
    assert "el_hbm_calib" in ec.el_last_error()
    assert L.el_hbm_calib(ec.EL_CALIB_READ | 64, A, A, 1 << 20, None, 0, 0, None) == INVALID  # unknown policy bit
    assert L.el_hbm_calib(-1, A, A, 1 << 20, None, 0, 0, None) == INVALID
    assert L.el_hbm_calib(ec.EL_CALIB_WRITE, None, A, 0, None, 0, 0, None) == ec.EL_OK     # nothing to move
    policy = ec.EL_CALIB_NT_LOADS | ec.EL_CALIB_NT_STORES
    assert L.el_hbm_calib(ec.EL_CALIB_COPY | policy, A, A, 0, None, 0, 0, None) == ec.EL_OK


def test_grad_calls_reject_small_or_missing_workspace():
    L = ec.lib()
    t, b = tables(), bags()
    need = L.emb_grad_workspace_bytes(ref(t), ref(b))
    assert L.emb_grad_reduce_update(ref(t), ref(b), 0, A, ec.EL_BF16, ctypes.c_float(0.01), A, need - 1, None) == WORKSPACE
    assert "needed" in ec.el_last_error()
    assert L.emb_grad_reduce_update(ref(t), ref(b), 0, A, ec.EL_BF16, ctypes.c_float(0.01), 0, need, None) == WORKSPACE
    assert L.emb_grad_reduce_update(ref(t), ref(b), 0, A, ec.EL_BF16, ctypes.c_float(0.01), A + 64, need, None) == INVALID
    assert L.emb_grad_reduce_update(ref(t), ref(b), 0, A, 3, ctypes.c_float(0.01), A, need, None) == INVALID
    assert L.emb_grad_sort(ref(t), ref(b), 0, A, need, A, A, A, 0, A, None) == INVALID
    assert L.emb_grad_sort(ref(t), ref(b), 0, A, 16, A, A, A, A, A, None) == WORKSPACE
    assert L.el_validate_bags(ref(t), ref(b), 0, 0, None) == INVALID
    assert L.el_validate_bags(ref(t), ref(b), 0, A + 4, None) == INVALID


def test_noalloc_update_refuses_workspaces_beyond_its_scratch_on_the_host():
    """The no-alloc update checks its arguments and the workspace it would need against the
    static scratch before touching a GPU."""
    L = ec.lib()
    lr = ctypes.c_float(0.01)
    t, b = tables(), bags()  # 26 x 65536 lookups of 128-wide rows: above the scratch
    need = L.emb_grad_workspace_bytes(ref(t), ref(b))
    assert need > ec.EL_NOALLOC_SCRATCH_BYTES
    assert L.emb_grad_reduce_update_noalloc(ref(t), ref(b), 0, A, ec.EL_BF16, lr, None) == WORKSPACE
    assert "emb_grad_reduce_update_noalloc" in ec.el_last_error() and "scratch" in ec.el_last_error()
    assert L.emb_grad_reduce_update_noalloc(None, ref(b), 0, A, ec.EL_BF16, lr, None) == INVALID
    assert L.emb_grad_reduce_update_noalloc(ref(t), ref(b), 2, A, ec.EL_BF16, lr, None) == INVALID
    assert L.emb_grad_reduce_update_noalloc(ref(t), ref(b), 0, A, 7, lr, None) == INVALID
    assert L.emb_grad_reduce_update_noalloc(ref(t), ref(b), 0, A + 8, ec.EL_BF16, lr, None) == INVALID
    assert L.emb_grad_reduce_update_noalloc(ref(t), ref(bags(B=0, nnz=0)), 0, A, ec.EL_BF16, lr, None) == ec.EL_OK


def test_table_row_limits():
    L = ec.lib()
    t = ec.ElTables(A, A, 1 << 32, 1, 128, ec.EL_F32)  # 2^32 rows: keys would not fit 32 bits
    assert L.emb_bag_fwd(ref(t), ref(bags(F=1)), 0, A, ec.EL_F32, None) == INVALID
    t = tables(max_rows=26 * 100_000 + 1)  # a table larger than all rows together
    assert L.emb_bag_fwd(ref(t), ref(bags()), 0, A, ec.EL_F32, None) == INVALID
    assert b"max_rows" in L.el_last_error()


def test_dense_layer_calls_reject_on_the_host():
    L = ec.lib()
    f = L.el_linear_fwd
    ok = dict(x=A, ldx=1024, M=65536, K=1024, w=A, bias=A, N=1024, act=ec.EL_ACT_RELU, y=A,
              ldy=1024, dt=ec.EL_BF16)

    def fwd(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["ldx"], a["M"], a["K"], a["w"], a["bias"], a["N"], a["act"], a["y"],
                 a["ldy"], a["dt"], None)

    assert fwd(K=13) == UNSUPPORTED                 # K not a multiple of 8
    assert fwd(N=12, ldy=16) == UNSUPPORTED         # N neither 1 nor a multiple of 8
    assert fwd(N=1, K=4096, ldx=4096) == UNSUPPORTED  # one-output layers take K <= 2048
    assert fwd(dt=ec.EL_F32) == UNSUPPORTED
    assert fwd(ldx=1000) == INVALID                 # ldx < K
    assert fwd(x=A + 8) == INVALID                  # misaligned x
    assert fwd(w=0) == INVALID
    assert fwd(act=5) == INVALID
    assert fwd(bias=A + 4) == INVALID
    assert fwd(ldy=1000) == INVALID
    assert "el_linear_fwd" in ec.el_last_error()
    assert fwd(M=0, x=0, y=0) == ec.EL_OK           # empty batch: nothing enqueued

    need = L.el_linear_bwd_workspace_bytes(65536, 1024, 1024)
    assert need >= 8 * 1024 * 1024 * 4              # fp32 partial weight gradients of the splits
    assert L.el_linear_bwd_workspace_bytes(65536, 1024, 1024) == need  # pure
    assert L.el_linear_bwd_workspace_bytes(-1, 1024, 1024) == 0
    b = L.el_linear_bwd
    args = [A, 1024, 65536, 1024, A, 1024, A, 1024, A, 1024, 0, A, A, ec.EL_BF16]
    assert b(*args, A, need - 1, None) == WORKSPACE
    assert b(*args, 0, need, None) == WORKSPACE
    assert b(*args[:10], 2, *args[11:], A, need, None) == INVALID        # unknown flag
    assert b(*args[:8], None, 1024, ec.EL_LINEAR_DX_RELU_MASK, *args[11:], A, need, None) == INVALID
    assert b(*args[:11], 0, *args[12:], A, need, None) == INVALID        # null dw
    assert "el_linear_bwd" in ec.el_last_error()

    assert L.el_relu_bwd(A, A, A, 100, 12, 16, ec.EL_BF16, None) == UNSUPPORTED
    assert L.el_relu_bwd(A, A, A + 2, 100, 16, 16, ec.EL_BF16, None) == INVALID
    assert L.el_relu_bwd(A, A, A, 0, 16, 16, ec.EL_BF16, None) == ec.EL_OK
    assert L.el_bce_workspace_bytes(65536) == 256 * 8
    assert L.el_bce_workspace_bytes(0) == 0
    assert L.el_bce_logits(A, 1, A, 0, ec.EL_BF16, A, A, 1, A, 8, None) == INVALID
    assert L.el_bce_logits(A, 1, A, 16, ec.EL_F32, A, A, 1, A, 8, None) == UNSUPPORTED
    assert L.el_bce_logits(A, 1, 0, 16, ec.EL_BF16, A, A, 1, A, 8, None) == INVALID
    assert L.el_bce_logits(A, 1, A, 1000, ec.EL_BF16, A, A, 1, A, 8, None) == WORKSPACE
    assert L.el_bce_logits(A, 1, A, 1000, ec.EL_BF16, A, A, 1, 0, 64, None) == WORKSPACE
    assert L.el_sgd_dense(A, A, ec.EL_BF16, A, -1, ctypes.c_float(0.01), None) == INVALID
    assert L.el_sgd_dense(A, A, 9, A, 10, ctypes.c_float(0.01), None) == UNSUPPORTED
    assert L.el_sgd_dense(A, A, ec.EL_BF16, A, 0, ctypes.c_float(0.01), None) == ec.EL_OK
