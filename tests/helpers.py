"""Shared helpers of the GPU parity tests: conversions between torch tensors and the
oracle's numpy buffers, the error measure, and sub-problem extraction for full-size
workloads (argument marshalling only; no arithmetic of the method lives here)."""
import numpy as np
import torch

NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}

# Tolerances: fp32 results within 1e-5 and bf16 / fp16 results within 2e-2 of the oracle,
# as relative errors err_i = |g_i - r_i| / max(|r_i|, rms(r)) (the rms floor keeps
# near-zero dot products from dominating); index / sort / segment outputs and hotness-1
# gathers are compared bit for bit.
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}


def to_np(t: torch.Tensor) -> np.ndarray:
    """Oracle layout of a tensor: float32 / float16 arrays, bf16 as raw uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_np(a: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    if dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def widen(a: np.ndarray, name: str) -> np.ndarray:
    if name == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref * ref))
    scale = np.maximum(np.abs(ref), rms)
    scale[scale == 0] = 1.0
    return float(np.max(np.abs(got - ref) / scale))


def assert_close(got: torch.Tensor, ref_np: np.ndarray, name: str, what: str):
    g = widen(to_np(got), name)
    r = widen(ref_np, name)
    assert not np.any(np.isnan(g)), f"{what}: NaN in GPU result"
    err = rel_err(g, r)
    assert err <= TOL[name], f"{what}: relative error {err:.3e} > {TOL[name]:.0e}"
    return err


def assert_bits(got: torch.Tensor, ref_np: np.ndarray, what: str):
    g = to_np(got)
    assert g.shape == ref_np.shape, f"{what}: shape {g.shape} vs {ref_np.shape}"
    assert g.dtype.itemsize == ref_np.dtype.itemsize, f"{what}: element sizes differ"
    gv = np.ascontiguousarray(g).reshape(-1).view(f"u{g.dtype.itemsize}")
    rv = np.ascontiguousarray(ref_np).reshape(-1).view(f"u{ref_np.dtype.itemsize}")
    diff = np.nonzero(gv != rv)[0]
    assert diff.size == 0, f"{what}: {diff.size} elements differ, first at flat index {diff[0]}"


def sub_batch(indices: np.ndarray, offsets: np.ndarray, F: int, B: int, samples: np.ndarray):
    """CSR of the bags of the chosen samples only (same tables), as (indices, offsets, B')."""
    parts, lens = [], []
    for t in range(F):
        for b in samples:
            g = t * B + int(b)
            s, e = int(offsets[g]), int(offsets[g + 1])
            parts.append(indices[s:e])
            lens.append(e - s)
    idx = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return idx, off, len(samples)


def compact_tables(W_dev: torch.Tensor, row_offset: np.ndarray, indices: np.ndarray,
                   offsets: np.ndarray, F: int, B: int):
    """Restrict a problem to the rows it looks up.  Each table keeps its looked-up rows in
    ascending order, so the renumbering preserves row order (and therefore the sorted
    order of the lookups).  Returns (W_compact numpy, row_offset_c, indices_c, global_rows)
    where global_rows[i] is the original joint-table row of compact row i."""
    new_idx = np.empty_like(indices)
    rows_all, ro_c = [], [0]
    for t in range(F):
        s, e = int(offsets[t * B]), int(offsets[(t + 1) * B])
        local = indices[s:e].astype(np.int64)
        u = np.unique(local)
        new_idx[s:e] = np.searchsorted(u, local).astype(np.int32)
        rows_all.append(u + int(row_offset[t]))
        ro_c.append(ro_c[-1] + u.size)
    global_rows = np.concatenate(rows_all) if rows_all else np.zeros(0, np.int64)
    sel = torch.from_numpy(global_rows).to(W_dev.device)
    Wc = to_np(W_dev.index_select(0, sel))
    return Wc, np.array(ro_c, np.int64), new_idx, global_rows
