"""Python binding of libembcore (the C ABI in ``include/embcore.h``).

Argument marshalling only: torch tensors are passed as raw device pointers plus sizes,
on torch's current HIP stream unless a stream is given.  Every step of the computation
runs in the library's HIP kernels; if the library is missing this module raises at load.
Function names and argument order follow the C ABI.
"""
import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libembcore.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "embcore.h")

EL_OK, EL_ERR_INVALID_ARG, EL_ERR_UNSUPPORTED, EL_ERR_WORKSPACE, EL_ERR_HIP = range(5)
EL_F32, EL_F16, EL_BF16 = 0, 1, 2
EL_FLAG_HASH_INDICES = 1
EL_ACT_NONE, EL_ACT_RELU = 0, 1
EL_LINEAR_DX_RELU_MASK = 1
EL_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/embcore.h
EL_CALIB_READ, EL_CALIB_WRITE, EL_CALIB_COPY, EL_CALIB_READ3_WRITE1, EL_CALIB_GATHER, EL_CALIB_GATHER_READ = range(6)
EL_CALIB_NT_LOADS, EL_CALIB_NT_STORES = 16, 32  # cache-policy bits OR-ed into the mode

_DTYPE = {torch.float32: EL_F32, torch.float16: EL_F16, torch.bfloat16: EL_BF16}


class EmbcoreError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class ElTables(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("row_offset", ctypes.c_void_p),
                ("total_rows", ctypes.c_int64), ("num_tables", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("dtype", ctypes.c_int), ("max_rows", ctypes.c_int64)]


class ElBags(ctypes.Structure):
    _fields_ = [("indices", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("nnz", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with embedding_lookup_feature_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
        T, Bg = ctypes.POINTER(ElTables), ctypes.POINTER(ElBags)
        L.emb_bag_fwd.argtypes = [T, Bg, u32, vp, ctypes.c_int, vp]
        L.dot_interact_fwd.argtypes = [vp, vp, ctypes.c_int, i32, i32, i32, vp, ctypes.c_int, i32, vp]
        L.emb_dot_fwd.argtypes = [T, Bg, u32, vp, ctypes.c_int, vp, vp, i32, vp]
        L.emb_dot_bwd.argtypes = [T, Bg, u32, vp, ctypes.c_int, vp, i32, vp, vp, ctypes.c_int, vp]
        L.dot_interact_bwd.argtypes = [vp, vp, ctypes.c_int, i32, i32, i32, vp, ctypes.c_int, i32,
                                       vp, vp, ctypes.c_int, vp]
        L.cat_interact_fwd.argtypes = [vp, vp, ctypes.c_int, i32, i32, i32, vp, ctypes.c_int, i32, vp]
        L.cat_interact_bwd.argtypes = [vp, ctypes.c_int, i32, i32, i32, i32, vp, vp, ctypes.c_int, vp]
        L.emb_cat_fwd.argtypes = [T, Bg, u32, vp, ctypes.c_int, vp, i32, vp]
        L.emb_grad_workspace_bytes.argtypes = [T, Bg]
        L.emb_grad_workspace_bytes.restype = ctypes.c_size_t
        L.emb_grad_reduce_update.argtypes = [T, Bg, u32, vp, ctypes.c_int, f32, vp, ctypes.c_size_t, vp]
        L.emb_grad_reduce_update_noalloc.argtypes = [T, Bg, u32, vp, ctypes.c_int, f32, vp]
        L.emb_grad_prepare.argtypes = [T, Bg, u32, vp, ctypes.c_size_t, vp]
        L.emb_grad_apply.argtypes = [T, Bg, u32, vp, ctypes.c_int, f32, vp, ctypes.c_size_t, vp]
        L.emb_grad_sort.argtypes = [T, Bg, u32, vp, ctypes.c_size_t, vp, vp, vp, vp, vp, vp]
        L.el_validate_bags.argtypes = [T, Bg, u32, vp, vp]
        sz = ctypes.c_size_t
        L.el_linear_fwd.argtypes = [vp, i32, i32, i32, vp, vp, i32, u32, vp, i32, ctypes.c_int, vp]
        L.el_linear_bwd_workspace_bytes.argtypes = [i32, i32, i32]
        L.el_linear_bwd_workspace_bytes.restype = sz
        L.el_linear_bwd.argtypes = [vp, i32, i32, i32, vp, i32, vp, i32, vp, i32, u32, vp, vp,
                                    ctypes.c_int, vp, sz, vp]
        L.el_relu_bwd.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_int, vp]
        L.el_bce_workspace_bytes.argtypes = [i32]
        L.el_bce_workspace_bytes.restype = sz
        L.el_bce_logits.argtypes = [vp, i32, vp, i32, ctypes.c_int, vp, vp, i32, vp, sz, vp]
        L.el_sgd_dense.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int64, f32, vp]
        L.el_hbm_calib.argtypes = [i32, vp, vp, ctypes.c_size_t, vp, ctypes.c_int64, i32, vp]
        L.el_hbm_calib.restype = ctypes.c_int
        L.el_last_error.restype = ctypes.c_char_p
        L.el_version.restype = ctypes.c_int
        for name in ("emb_bag_fwd", "dot_interact_fwd", "emb_dot_fwd", "dot_interact_bwd", "emb_dot_bwd",
                     "cat_interact_fwd", "cat_interact_bwd", "emb_cat_fwd",
                     "emb_grad_reduce_update", "emb_grad_reduce_update_noalloc",
                     "emb_grad_prepare", "emb_grad_apply",
                     "emb_grad_sort", "el_validate_bags", "el_linear_fwd", "el_linear_bwd",
                     "el_relu_bwd", "el_bce_logits", "el_sgd_dense"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions():
    """Names of the functions `include/embcore.h` declares."""
    text = open(HEADER).read()
    return re.findall(r"EL_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def _check(status: int):
    if status != EL_OK:
        raise EmbcoreError(status, el_last_error())


def el_last_error() -> str:
    return lib().el_last_error().decode()


def el_version() -> int:
    return lib().el_version()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DTYPE:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


class Tables:
    """F embedding tables in one joint [total_rows, D] buffer; table t owns rows
    row_offset[t] .. row_offset[t+1]-1."""

    def __init__(self, weight: torch.Tensor, row_offset: torch.Tensor, total_rows: int = None,
                 max_rows: int = None):
        """max_rows: rows of the largest table; None reads it from row_offset (one copy to the
        host, here and not per call), 0 leaves it unknown."""
        if weight.dim() != 2 or row_offset.dtype != torch.int64 or row_offset.dim() != 1:
            raise ValueError("weight must be [total_rows, D]; row_offset int64 [F+1]")
        self.weight = weight
        self.row_offset = row_offset
        self.total_rows = int(weight.shape[0] if total_rows is None else total_rows)
        if max_rows is None:
            ro = row_offset.cpu()
            max_rows = int((ro[1:] - ro[:-1]).max()) if ro.numel() > 1 else 0
        self.max_rows = int(max_rows)
        self.c = ElTables(_dev(weight, "weight"), _dev(row_offset, "row_offset"), self.total_rows,
                          row_offset.numel() - 1, weight.shape[1], _dtype(weight, "weight"), self.max_rows)

    @property
    def num_tables(self):
        return self.c.num_tables

    @property
    def dim(self):
        return self.c.dim


class Bags:
    """CSR lookups over F*B table-major bags (bag t*B + b)."""

    def __init__(self, indices: torch.Tensor, offsets: torch.Tensor, batch: int, nnz: int = None):
        if indices.dtype != torch.int32 or offsets.dtype != torch.int32:
            raise ValueError("indices and offsets must be int32")
        self.indices = indices
        self.offsets = offsets
        self.batch = int(batch)
        self.nnz = int(indices.numel() if nnz is None else nnz)
        ip = _dev(indices, "indices") if indices.numel() else 0
        self.c = ElBags(ip, _dev(offsets, "offsets"), self.batch, self.nnz)


def emb_bag_fwd(tables: Tables, bags: Bags, emb_out: torch.Tensor, hash_indices=False, stream=None):
    """emb_out[b][t] = sum of the rows of bag (t, b); emb_out is [B, F, D]."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    _check(lib().emb_bag_fwd(ctypes.byref(tables.c), ctypes.byref(bags.c), flags,
                             _dev(emb_out, "emb_out"), _dtype(emb_out, "emb_out"), _stream(stream)))
    return emb_out


def dot_interact_fwd(x0: torch.Tensor, emb: torch.Tensor, out: torch.Tensor, stream=None):
    """out[b] = [x0[b] | strict-lower pair dot products | 0 pad]; out is [B, out_stride]."""
    B, F, D = emb.shape
    _check(lib().dot_interact_fwd(_dev(x0, "x0"), _dev(emb, "emb"), _dtype(emb, "emb"), B, F, D,
                                  _dev(out, "out"), _dtype(out, "out"), out.shape[1], _stream(stream)))
    return out


def emb_dot_fwd(tables: Tables, bags: Bags, x0: torch.Tensor, out: torch.Tensor,
                emb_out: torch.Tensor = None, hash_indices=False, stream=None):
    """emb_bag_fwd into emb_out followed by dot_interact_fwd into out, in one call (bit-identical
    results); emb_out may be None when the pooled vectors are not needed."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    ep = _dev(emb_out, "emb_out") if emb_out is not None else None
    if emb_out is not None and emb_out.dtype != x0.dtype:
        raise ValueError("emb_out must have the activation dtype of x0")
    _check(lib().emb_dot_fwd(ctypes.byref(tables.c), ctypes.byref(bags.c), flags, _dev(x0, "x0"),
                             _dtype(x0, "x0"), ep, _dev(out, "out"), out.shape[1], _stream(stream)))
    return out


def dot_interact_bwd(x0, emb, dout, dx0, demb, stream=None):
    """Interaction gradients for upstream gradient dout [B, out_stride]."""
    B, F, D = emb.shape
    _check(lib().dot_interact_bwd(_dev(x0, "x0"), _dev(emb, "emb"), _dtype(emb, "emb"), B, F, D,
                                  _dev(dout, "dout"), _dtype(dout, "dout"), dout.shape[1],
                                  _dev(dx0, "dx0"), _dev(demb, "demb"), _dtype(demb, "demb"),
                                  _stream(stream)))
    return dx0, demb


def emb_dot_bwd(tables: Tables, bags: Bags, x0: torch.Tensor, dout: torch.Tensor,
                dx0: torch.Tensor, demb: torch.Tensor, hash_indices=False, stream=None):
    """emb_bag_fwd followed by dot_interact_bwd in one call (bit-identical results), the pooled
    vectors rebuilt from the tables and never stored."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    if dout.dtype != x0.dtype:
        raise ValueError("dout must have the activation dtype of x0")
    _check(lib().emb_dot_bwd(ctypes.byref(tables.c), ctypes.byref(bags.c), flags, _dev(x0, "x0"),
                             _dtype(x0, "x0"), _dev(dout, "dout"), dout.shape[1], _dev(dx0, "dx0"),
                             _dev(demb, "demb"), _dtype(demb, "demb"), _stream(stream)))
    return dx0, demb


def emb_grad_workspace_bytes(tables: Tables, bags: Bags) -> int:
    return int(lib().emb_grad_workspace_bytes(ctypes.byref(tables.c), ctypes.byref(bags.c)))


def alloc_workspace(tables: Tables, bags: Bags, device=None) -> torch.Tensor:
    """A byte tensor large enough for the gradient path (torch allocations are 256-aligned)."""
    n = max(emb_grad_workspace_bytes(tables, bags), 256)
    return torch.empty(n, dtype=torch.uint8, device=device or tables.weight.device)


def cat_interact_fwd(x0: torch.Tensor, emb: torch.Tensor, out: torch.Tensor, stream=None):
    """--interaction_op cat: out[b] = [x0[b] | emb[b][0] | ... | emb[b][F-1] | 0 pad]."""
    B, F, D = emb.shape
    _check(lib().cat_interact_fwd(_dev(x0, "x0"), _dev(emb, "emb"), _dtype(emb, "emb"), B, F, D,
                                  _dev(out, "out"), _dtype(out, "out"), out.shape[1], _stream(stream)))
    return out


def cat_interact_bwd(dout: torch.Tensor, dx0: torch.Tensor, demb: torch.Tensor, stream=None):
    """Gradients of the cat interaction: dx0 = dout[:, :D], demb[:, t] = dout[:, D(1+t):D(2+t)]."""
    B, F, D = demb.shape
    _check(lib().cat_interact_bwd(_dev(dout, "dout"), _dtype(dout, "dout"), B, F, D, dout.shape[1],
                                  _dev(dx0, "dx0"), _dev(demb, "demb"), _dtype(demb, "demb"),
                                  _stream(stream)))


def emb_cat_fwd(tables: Tables, bags: Bags, x0: torch.Tensor, out: torch.Tensor, hash_indices=False,
                stream=None):
    """emb_bag_fwd + cat_interact_fwd in one call: pooled vectors written straight into their
    blocks of the output rows."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    _check(lib().emb_cat_fwd(ctypes.byref(tables.c), ctypes.byref(bags.c), flags, _dev(x0, "x0"),
                             _dtype(x0, "x0"), _dev(out, "out"), out.shape[1], _stream(stream)))
    return out


def hbm_calib(mode: int, src, dst: torch.Tensor, nbytes: int = 0, idx: torch.Tensor = None,
              row_bytes: int = 0, stream=None):
    """One HBM calibration kernel (EL_CALIB_*): `nbytes` of streaming traffic, or the rows
    idx of the table `src` gathered into `dst` (row_bytes each)."""
    sp = _dev(src, "src") if src is not None else None
    ip = _dev(idx, "idx") if idx is not None else None
    nrows = idx.numel() if idx is not None else 0
    _check(lib().el_hbm_calib(mode, sp, _dev(dst, "dst"), nbytes, ip, nrows, row_bytes, _stream(stream)))


def emb_grad_reduce_update(tables: Tables, bags: Bags, demb: torch.Tensor, lr: float,
                           workspace: torch.Tensor, hash_indices=False, stream=None):
    """Sparse SGD: every looked-up row r gets W[r] -= lr * (sum of its lookups' gradients)."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    _check(lib().emb_grad_reduce_update(ctypes.byref(tables.c), ctypes.byref(bags.c), flags,
                                        _dev(demb, "demb"), _dtype(demb, "demb"), float(lr),
                                        _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))


def emb_grad_reduce_update_noalloc(tables: Tables, bags: Bags, demb: torch.Tensor, lr: float,
                                   hash_indices=False, stream=None):
    """emb_grad_reduce_update with the library's static per-GPU scratch as workspace (for
    callers that cannot allocate); workspaces above EL_NOALLOC_SCRATCH_BYTES are refused."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    _check(lib().emb_grad_reduce_update_noalloc(ctypes.byref(tables.c), ctypes.byref(bags.c), flags,
                                                _dev(demb, "demb"), _dtype(demb, "demb"), float(lr),
                                                _stream(stream)))


def emb_grad_prepare(tables: Tables, bags: Bags, workspace: torch.Tensor, hash_indices=False,
                     stream=None):
    """First half of emb_grad_reduce_update: sort the lookups by row into `workspace`."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    _check(lib().emb_grad_prepare(ctypes.byref(tables.c), ctypes.byref(bags.c), flags,
                                  _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))


def emb_grad_apply(tables: Tables, bags: Bags, demb: torch.Tensor, lr: float, workspace: torch.Tensor,
                   hash_indices=False, stream=None):
    """Second half: segment reduce + SGD from the lookups emb_grad_prepare sorted."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    _check(lib().emb_grad_apply(ctypes.byref(tables.c), ctypes.byref(bags.c), flags,
                                _dev(demb, "demb"), _dtype(demb, "demb"), float(lr),
                                _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))


def emb_grad_sort(tables: Tables, bags: Bags, workspace: torch.Tensor, sorted_rows, bag_ids,
                  unique_rows, seg_offsets, num_unique, hash_indices=False, stream=None):
    """The sort / segment stage of the gradient path (int32 tensors hold uint32 values)."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    _check(lib().emb_grad_sort(ctypes.byref(tables.c), ctypes.byref(bags.c), flags,
                               _dev(workspace, "workspace"), workspace.numel(),
                               _dev(sorted_rows, "sorted_rows"), _dev(bag_ids, "bag_ids"),
                               _dev(unique_rows, "unique_rows"), _dev(seg_offsets, "seg_offsets"),
                               _dev(num_unique, "num_unique"), _stream(stream)))


def el_validate_bags(tables: Tables, bags: Bags, bad_count: torch.Tensor, hash_indices=False,
                     stream=None):
    """bad_count (int64 [1]) := number of CSR defects / out-of-range indices."""
    flags = EL_FLAG_HASH_INDICES if hash_indices else 0
    _check(lib().el_validate_bags(ctypes.byref(tables.c), ctypes.byref(bags.c), flags,
                                  _dev(bad_count, "bad_count"), _stream(stream)))
    return bad_count


# ----------------------------------------------------------------------------------------
# dense layers, logistic loss, dense SGD
# ----------------------------------------------------------------------------------------

def _rows(t: torch.Tensor, name: str):
    """(pointer, rows, row stride) of a 2-D tensor whose rows may be strided (last dim dense)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.data_ptr(), t.shape[0], t.stride(0)


def linear_fwd(x: torch.Tensor, w: torch.Tensor, bias, y: torch.Tensor, relu: bool, stream=None):
    """y[:, :N] = act(x[:, :K] @ w.T + bias) with w [N, K]; x, y may be row-strided views."""
    xp, M, ldx = _rows(x, "x")
    N, K = w.shape
    yp, My, ldy = _rows(y, "y")
    if My != M or y.dtype != x.dtype or w.dtype != x.dtype:
        raise ValueError("x, w, y must share the dtype; y must have M rows")
    bp = _dev(bias, "bias") if bias is not None else None
    _check(lib().el_linear_fwd(xp, ldx, M, K, _dev(w, "w"), bp, N,
                               EL_ACT_RELU if relu else EL_ACT_NONE, yp, ldy, _dtype(x, "x"),
                               _stream(stream)))
    return y


def linear_bwd_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().el_linear_bwd_workspace_bytes(M, K, N))


def linear_bwd(x: torch.Tensor, w: torch.Tensor, dz: torch.Tensor, dw: torch.Tensor,
               db: torch.Tensor, dx: torch.Tensor = None, relu_mask: bool = False,
               workspace: torch.Tensor = None, stream=None):
    """dw = dz^T x, db = dz.sum(0) (fp32) and, when dx is given, dx = dz @ w (times
    1[x > 0] with relu_mask).  workspace: bytes >= linear_bwd_workspace_bytes(M, K, N)."""
    xp, M, ldx = _rows(x, "x")
    N, K = w.shape
    zp, Mz, ldz = _rows(dz, "dz")
    if Mz != M:
        raise ValueError("dz must have M rows")
    dxp, lddx = (None, K)
    if dx is not None:
        dxp, Mx, lddx = _rows(dx, "dx")
        if Mx != M:
            raise ValueError("dx must have M rows")
    need = linear_bwd_workspace_bytes(M, K, N)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wp = _dev(workspace, "workspace") if workspace is not None else None
    wn = workspace.numel() if workspace is not None else 0
    _check(lib().el_linear_bwd(xp, ldx, M, K, _dev(w, "w"), N, zp, ldz, dxp, lddx,
                               EL_LINEAR_DX_RELU_MASK if relu_mask else 0, _dev(dw, "dw"),
                               _dev(db, "db"), _dtype(x, "x"), wp, wn, _stream(stream)))
    return dx, dw, db


def relu_bwd(dy: torch.Tensor, y: torch.Tensor, dz: torch.Tensor, stream=None):
    """dz = dy * 1[y > 0] (the ReLU derivative from its output)."""
    M, N = dy.shape
    if y.shape != dy.shape or dz.shape != dy.shape:
        raise ValueError("dy, y, dz must have one shape")
    _check(lib().el_relu_bwd(_dev(dy, "dy"), _dev(y, "y"), _dev(dz, "dz"), M, N, N,
                             _dtype(dy, "dy"), _stream(stream)))
    return dz


def bce_workspace_bytes(M: int) -> int:
    return int(lib().el_bce_workspace_bytes(M))


def bce_logits(z: torch.Tensor, labels: torch.Tensor, loss: torch.Tensor, dz: torch.Tensor,
               workspace: torch.Tensor = None, stream=None):
    """loss[0] = batch-mean logistic loss of logits z ([M] or [M, 1] view), dz = dloss/dz.
    workspace: bytes >= bce_workspace_bytes(M) (allocated here when not given)."""
    M = labels.numel()
    if workspace is None:
        workspace = torch.empty(max(8, bce_workspace_bytes(M)), dtype=torch.uint8, device=z.device)
    ldz = z.stride(0) if z.dim() >= 1 else 1
    lddz = dz.stride(0) if dz.dim() >= 1 else 1
    if not (z.is_cuda and dz.is_cuda):
        raise ValueError("z and dz must be device tensors")
    _check(lib().el_bce_logits(z.data_ptr(), ldz, _dev(labels, "labels"), M, _dtype(z, "z"),
                               _dev(loss, "loss"), dz.data_ptr(), lddz, _dev(workspace, "workspace"),
                               workspace.numel(), _stream(stream)))
    return loss, dz


def sgd_dense(master: torch.Tensor, grad: torch.Tensor, lr: float, copy: torch.Tensor = None,
              stream=None):
    """master -= lr * grad (fp32); copy = master in the copy's 16-bit dtype."""
    cp = _dev(copy, "copy") if copy is not None else None
    cd = _dtype(copy, "copy") if copy is not None else EL_BF16
    _check(lib().el_sgd_dense(_dev(master, "master"), cp, cd, _dev(grad, "grad"), master.numel(),
                              float(lr), _stream(stream)))
