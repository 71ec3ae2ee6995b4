"""numpy front end of the C oracle (``emb_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the benchmark's
CPU-baseline leg; the product path never loads it.

Buffers are numpy arrays.  A 16-bit float buffer is a ``np.uint16`` array of raw bit
patterns (bf16) or a ``np.float16`` array (fp16); every function takes the dtype name of
each float buffer explicitly ("f32", "f16", "bf16", "f64").  Every function follows the
page "DLRM For PyTorch" (§Model architecture; §Command-line options for --hash_indices and
--lr); the C source states the definition each one writes out.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_CODES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "f64": np.float64}
_ERRORS = {
    -1: "unknown dtype",
    -2: "index outside its table",
    -3: "offsets not monotone or not starting at 0",
    -4: "out of memory",
    -5: "bad shape",
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the oracle library, compiling it first if it is missing or stale."""
    global _lib
    if _lib is None:
        if (not os.path.exists(_build.LIB)
                or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _lib = _configure(ctypes.CDLL(_build.LIB))
    return _lib


def _configure(L):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.oracle_emb_bag_fwd.argtypes = [vp, i32, vp, i32, i32, vp, vp, i32, i32, vp, i32]
    L.oracle_dot_interact_fwd.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, i32]
    L.oracle_dot_interact_bwd.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, i32, vp, vp, i32]
    L.oracle_cat_interact_fwd.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, i32]
    L.oracle_cat_interact_bwd.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, i32]
    L.oracle_grad_sort.argtypes = [vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    L.oracle_grad_reduce_update.argtypes = [vp, i32, vp, i32, i32, vp, vp, i32, i32, vp, i32,
                                            ctypes.c_float]
    L.oracle_round_f64.argtypes = [vp, i64, i32, vp]
    L.oracle_widen.argtypes = [vp, i64, i32, vp]
    L.oracle_linear_fwd.argtypes = [vp, i32, i32, i32, i32, vp, i32, i32, vp, i32, vp, i32, i32]
    L.oracle_linear_bwd.argtypes = [vp, i32, i32, i32, i32, vp, i32, i32, vp, i32, i32, vp, vp,
                                    i32, vp, vp, i32]
    L.oracle_relu_bwd.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    L.oracle_bce_logits.argtypes = [vp, i32, vp, i32, vp, vp, i32]
    L.oracle_sgd_dense.argtypes = [vp, vp, i64, ctypes.c_float, vp, i32]
    for name in ("oracle_emb_bag_fwd", "oracle_dot_interact_fwd", "oracle_dot_interact_bwd",
                 "oracle_cat_interact_fwd", "oracle_cat_interact_bwd",
                 "oracle_grad_sort", "oracle_grad_reduce_update", "oracle_linear_fwd",
                 "oracle_linear_bwd", "oracle_relu_bwd", "oracle_bce_logits", "oracle_sgd_dense", "oracle_version"):
        getattr(L, name).restype = ctypes.c_int
    L.oracle_round_f64.restype = None
    L.oracle_widen.restype = None
    return L


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


def _as(a, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != _NP[dtype]:
        raise TypeError(f"buffer has numpy dtype {a.dtype}, expected {_NP[dtype]} for {dtype}")
    return a


def empty(shape, dtype: str) -> np.ndarray:
    """Output buffer filled with all-ones bytes (a NaN pattern), so that any element an
    oracle function fails to write shows up."""
    a = np.empty(shape, dtype=_NP[dtype])
    a.view(np.uint8)[...] = 0xFF
    return a


def round_from_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once, to nearest even, into `dtype` (raw bits for bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = empty(x.shape, dtype)
    lib().oracle_round_f64(_ptr(x), x.size, _CODES[dtype], _ptr(out))
    return out


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a buffer stored in `dtype`."""
    x = _as(x, dtype)
    out = np.zeros(x.shape, dtype=np.float64)
    lib().oracle_widen(_ptr(x), x.size, _CODES[dtype], _ptr(out))
    return out


def emb_bag_fwd(W, w_dtype, row_offset, indices, offsets, batch, dim, out_dtype, hash_indices=False):
    """Sum-pooled embedding bags; returns emb [B][F][D] in `out_dtype`."""
    W = _as(W, w_dtype)
    row_offset = np.ascontiguousarray(row_offset, dtype=np.int64)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    F = row_offset.size - 1
    out = empty((batch, F, dim), out_dtype)
    _check(lib().oracle_emb_bag_fwd(_ptr(W), _CODES[w_dtype], _ptr(row_offset), F, dim,
                                    _ptr(indices), _ptr(offsets), batch, int(hash_indices),
                                    _ptr(out), _CODES[out_dtype]))
    return out


def dot_interact_fwd(x0, emb, in_dtype, out_dtype, out_stride):
    """[x0 | strict-lower pair dots | zero pad] per sample; returns out [B][out_stride]."""
    x0 = _as(x0, in_dtype)
    emb = _as(emb, in_dtype)
    B, F, D = emb.shape
    out = empty((B, out_stride), out_dtype)
    _check(lib().oracle_dot_interact_fwd(_ptr(x0), _ptr(emb), _CODES[in_dtype], B, F, D,
                                         _ptr(out), _CODES[out_dtype], out_stride))
    return out


def dot_interact_bwd(x0, emb, in_dtype, dout, dout_dtype, grad_dtype):
    """Gradients of the interaction; returns (dx0 [B][D], demb [B][F][D]) in `grad_dtype`."""
    x0 = _as(x0, in_dtype)
    emb = _as(emb, in_dtype)
    dout = _as(dout, dout_dtype)
    B, F, D = emb.shape
    dx0 = empty((B, D), grad_dtype)
    demb = empty((B, F, D), grad_dtype)
    _check(lib().oracle_dot_interact_bwd(_ptr(x0), _ptr(emb), _CODES[in_dtype], B, F, D,
                                         _ptr(dout), _CODES[dout_dtype], dout.shape[1],
                                         _ptr(dx0), _ptr(demb), _CODES[grad_dtype]))
    return dx0, demb


def cat_interact_fwd(x0, emb, in_dtype, out_dtype, out_stride):
    """--interaction_op cat: [x0 | emb[0] | ... | emb[F-1] | zero pad] per sample; returns
    out [B][out_stride]."""
    x0 = _as(x0, in_dtype)
    emb = _as(emb, in_dtype)
    B, F, D = emb.shape
    out = empty((B, out_stride), out_dtype)
    _check(lib().oracle_cat_interact_fwd(_ptr(x0), _ptr(emb), _CODES[in_dtype], B, F, D,
                                         _ptr(out), _CODES[out_dtype], out_stride))
    return out


def cat_interact_bwd(dout, dout_dtype, F, D, grad_dtype):
    """Gradients of the cat interaction (each vector's block of dout); returns
    (dx0 [B][D], demb [B][F][D]) in `grad_dtype`."""
    dout = _as(dout, dout_dtype)
    B, S = dout.shape
    dx0 = empty((B, D), grad_dtype)
    demb = empty((B, F, D), grad_dtype)
    _check(lib().oracle_cat_interact_bwd(_ptr(dout), _CODES[dout_dtype], B, F, D, S, _ptr(dx0),
                                         _ptr(demb), _CODES[grad_dtype]))
    return dx0, demb


def grad_sort(row_offset, indices, offsets, batch, hash_indices=False):
    """Stable sort of the lookups by global row, plus run-length segments.

    Returns a dict with sorted_rows, bag_ids, unique_rows, seg_offsets (uint32 arrays)."""
    row_offset = np.ascontiguousarray(row_offset, dtype=np.int64)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    F = row_offset.size - 1
    n = int(offsets[-1])
    sorted_rows = np.zeros(n, np.uint32)
    bag_ids = np.zeros(n, np.uint32)
    unique_rows = np.zeros(max(n, 1), np.uint32)
    seg_offsets = np.zeros(n + 1, np.uint32)
    num_unique = np.zeros(1, np.uint32)
    _check(lib().oracle_grad_sort(_ptr(row_offset), F, _ptr(indices), _ptr(offsets), batch,
                                  int(hash_indices), _ptr(sorted_rows), _ptr(bag_ids),
                                  _ptr(unique_rows), _ptr(seg_offsets), _ptr(num_unique)))
    U = int(num_unique[0])
    return {"sorted_rows": sorted_rows, "bag_ids": bag_ids, "unique_rows": unique_rows[:U],
            "seg_offsets": seg_offsets[:U + 1], "num_unique": U}


def grad_reduce_update(W, w_dtype, row_offset, indices, offsets, batch, demb, grad_dtype, lr,
                       hash_indices=False):
    """Sparse SGD row update; returns the updated copy of W (W itself is not modified)."""
    W = np.array(_as(W, w_dtype), copy=True)
    demb = _as(demb, grad_dtype)
    row_offset = np.ascontiguousarray(row_offset, dtype=np.int64)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    F = row_offset.size - 1
    D = W.shape[-1]
    _check(lib().oracle_grad_reduce_update(_ptr(W), _CODES[w_dtype], _ptr(row_offset), F, D,
                                           _ptr(indices), _ptr(offsets), batch,
                                           int(hash_indices), _ptr(demb), _CODES[grad_dtype],
                                           ctypes.c_float(lr)))
    return W


def linear_fwd(x, x_dtype, w, w_dtype, bias, relu, y_dtype, K=None, ldy=None):
    """Dense layer forward y = act(x[:, :K] w^T + bias); x [M][ldx], w [N][K], bias fp32 [N]
    or None.  Returns y [M][ldy] (columns past N untouched: the NaN fill of ``empty``)."""
    x = _as(x, x_dtype)
    w = _as(w, w_dtype)
    M, ldx = x.shape
    N, Kw = w.shape
    K = Kw if K is None else K
    assert K == Kw
    ldy = N if ldy is None else ldy
    y = empty((M, ldy), y_dtype)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _check(lib().oracle_linear_fwd(_ptr(x), _CODES[x_dtype], M, K, ldx, _ptr(w), _CODES[w_dtype],
                                   N, None if b is None else _ptr(b), int(bool(relu)), _ptr(y),
                                   _CODES[y_dtype], ldy))
    return y


def linear_bwd(x, x_dtype, w, w_dtype, dz, dz_dtype, dx_dtype=None, relu_mask=False,
               wgrad_dtype="f32"):
    """Dense layer backward from dz = dL/d(pre-activation) [M][ldz].

    Returns (dx [M][ldx] or None, dw [N][K], db [N]).  dx is computed when `dx_dtype` is given;
    with `relu_mask` it is multiplied by 1[x > 0] (the ReLU of the layer below)."""
    x = _as(x, x_dtype)
    w = _as(w, w_dtype)
    dz = _as(dz, dz_dtype)
    M, ldx = x.shape
    N, K = w.shape
    ldz = dz.shape[1]
    dx = None if dx_dtype is None else empty((M, ldx), dx_dtype)
    dw = empty((N, K), wgrad_dtype)
    db = empty((N,), wgrad_dtype)
    _check(lib().oracle_linear_bwd(_ptr(x), _CODES[x_dtype], M, K, ldx, _ptr(w), _CODES[w_dtype],
                                   N, _ptr(dz), _CODES[dz_dtype], ldz,
                                   _ptr(x) if relu_mask else None,
                                   None if dx is None else _ptr(dx),
                                   _CODES[dx_dtype or "f32"], _ptr(dw), _ptr(db),
                                   _CODES[wgrad_dtype]))
    return dx, dw, db


def relu_bwd(dy, y, dtype):
    """dz = dy * 1[y > 0] for a ReLU with output y; returns dz with dy's shape."""
    dy = _as(dy, dtype)
    y = _as(y, dtype)
    M, N = dy.shape
    dz = empty((M, N), dtype)
    _check(lib().oracle_relu_bwd(_ptr(dy), _ptr(y), _CODES[dtype], M, N, N, _ptr(dz)))
    return dz


def bce_logits(z, z_dtype, labels, dz_dtype):
    """Batch-mean logistic loss on logits z [M] (labels fp32 in {0,1}); returns (loss, dz)."""
    z = _as(z, z_dtype).reshape(-1)
    labels = np.ascontiguousarray(labels, dtype=np.float32).reshape(-1)
    loss = np.zeros(1, np.float64)
    dz = empty(z.shape, dz_dtype)
    _check(lib().oracle_bce_logits(_ptr(z), _CODES[z_dtype], _ptr(labels), z.size, _ptr(loss),
                                   _ptr(dz), _CODES[dz_dtype]))
    return float(loss[0]), dz


def sgd_dense(master, grad, lr, copy_dtype=None):
    """SGD on an fp32 master copy; returns (new master, 16-bit copy or None).  Inputs are
    not modified."""
    master = np.array(np.ascontiguousarray(master, dtype=np.float32), copy=True)
    grad = np.ascontiguousarray(grad, dtype=np.float32)
    copy = None if copy_dtype is None else empty(master.shape, copy_dtype)
    _check(lib().oracle_sgd_dense(_ptr(master), _ptr(grad), master.size, ctypes.c_float(lr),
                                  None if copy is None else _ptr(copy), _CODES[copy_dtype or "f32"]))
    return master, copy


def use_library(path):
    """Swap the loaded oracle library for another build of the same source (the test
    suite uses this to check that its pins reject deliberately broken builds).  Returns
    the previously loaded library so that `restore_library` can put it back."""
    global _lib
    prev = lib()
    _lib = _configure(ctypes.CDLL(path))
    return prev


def restore_library(prev):
    global _lib
    _lib = prev
