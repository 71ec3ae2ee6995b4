"""The no-alloc embedding update (emb_grad_reduce_update_noalloc, the library's static
per-GPU scratch as workspace) against the call that takes a caller-allocated workspace
(GPU).  Both run the same kernels, so the tables they update must agree bit for bit; the
updated rows are also checked against the oracle.  Two calls in a row, the second on a
smaller input: the scratch keeps the first call's bytes, which the second must not read."""
import numpy as np
import pytest
import torch

import embedding_lookup_feature_amd as elf
from embedding_lookup_feature_amd import synth
from oracle import oracle as orc
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def problem(batch, batch_id, rows=(20_000,) * 26, dim=128):
    wl = synth.WORKLOADS["train_step"].scaled(name=f"noalloc{batch}", batch=batch, rows=rows, dim=dim)
    W, ro = synth.make_tables(wl, DEV)
    idx, off = synth.make_indices(wl, DEV, batch_id=batch_id)
    demb = synth.make_demb(wl, DEV, batch_id=batch_id)
    return wl, W, ro, idx, off, demb


def test_noalloc_update_matches_the_workspace_call_twice_in_a_row():
    for batch, batch_id in ((12000, 0), (3001, 1)):  # the second input is smaller
        wl, W, ro, idx, off, demb = problem(batch, batch_id)
        tab_probe, bags = elf.Tables(W, ro), elf.Bags(idx, off, batch)
        assert elf.emb_grad_workspace_bytes(tab_probe, bags) <= elf.embcore.EL_NOALLOC_SCRATCH_BYTES
        W_ws, W_na = W.clone(), W.clone()
        t_ws, t_na = elf.Tables(W_ws, ro), elf.Tables(W_na, ro)
        ws = elf.alloc_workspace(t_ws, bags)
        ws.fill_(0x3C)
        elf.emb_grad_reduce_update(t_ws, bags, demb, wl.lr, ws)
        elf.emb_grad_reduce_update_noalloc(t_na, bags, demb, wl.lr)
        torch.cuda.synchronize()
        assert torch.equal(W_na.view(torch.int32), W_ws.view(torch.int32)), f"B={batch}: tables differ"
        ref = orc.grad_reduce_update(to_np(W), "f32", to_np(ro), to_np(idx), to_np(off), batch,
                                     to_np(demb), "bf16", wl.lr)
        keys = orc.grad_sort(to_np(ro), to_np(idx), to_np(off), batch)["unique_rows"].astype(np.int64)
        sel = torch.from_numpy(keys).to(DEV)
        assert_close(W_na[sel], ref[keys], "f32", f"B={batch} updated rows")
        untouched = torch.ones(W.shape[0], dtype=torch.bool, device=DEV)
        untouched[sel] = False
        assert torch.equal(W_na[untouched].view(torch.int32), W[untouched].view(torch.int32))


def test_noalloc_update_refuses_a_workspace_beyond_its_scratch():
    wl, W, ro, idx, off, demb = problem(65536, 0, rows=(100_000,) * 26)
    tab, bags = elf.Tables(W, ro), elf.Bags(idx, off, 65536)
    W0 = W.clone()
    with pytest.raises(elf.EmbcoreError) as e:
        elf.emb_grad_reduce_update_noalloc(tab, bags, demb, wl.lr)
    assert e.value.status == elf.embcore.EL_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(W.view(torch.int32), W0.view(torch.int32))
