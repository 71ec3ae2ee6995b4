"""Checkpoint and resume (GPU): the model state is the caller's buffers (the embedding tables,
and for the whole model the MLPs' fp32 master weights and their 16-bit copies), so a
checkpoint is those bytes plus the step count.  Because every kernel on the path is
deterministic, k steps, a save to disk, a reload into freshly allocated buffers (new
Tables, new workspace, a new model object) and n more steps must end bit for bit where
k + n uninterrupted steps end.  The page's training script saves and reloads its model
(page "DLRM For PyTorch", §Command-line options: the checkpoint save and load paths);
this is the same contract for the state this library updates."""
import pytest
import torch

import embedding_lookup_feature_amd as elf
from embedding_lookup_feature_amd import dlrm, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bits(t):
    return t.contiguous().view(torch.uint8)


def core_workload():
    return synth.WORKLOADS["train_step"].scaled(name="ckpt-core", batch=1024, rows=(3000, 50, 1234, 777, 5),
                                                dim=64, bottom_mlp=(13, 64, 64))


def core_step(wl, tab, ws, i, out, emb, dx0, demb):
    """Forward, interaction backward and the sparse SGD update on batch i."""
    idx, off = synth.make_indices(wl, DEV, batch_id=i)
    bags = elf.Bags(idx, off, wl.batch)
    x0, G = synth.make_x0(wl, DEV, i), synth.make_dout(wl, DEV, i)
    elf.emb_dot_fwd(tab, bags, x0, out, emb)
    elf.dot_interact_bwd(x0, emb, G, dx0, demb)
    elf.emb_grad_reduce_update(tab, bags, demb, wl.lr, ws)


def core_buffers(wl):
    B, F, D = wl.batch, wl.num_tables, wl.dim
    act = synth.act_dtype(wl)
    return (torch.empty((B, wl.out_stride), dtype=act, device=DEV), torch.empty((B, F, D), dtype=act, device=DEV),
            torch.empty((B, D), dtype=act, device=DEV), torch.empty((B, F, D), dtype=act, device=DEV))


def workspace_for(wl, tab, steps):
    n = max(elf.emb_grad_workspace_bytes(tab, elf.Bags(*synth.make_indices(wl, DEV, batch_id=i), wl.batch))
            for i in steps)
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def test_core_step_resumes_bitwise_from_a_saved_table(tmp_path):
    wl = core_workload()
    K, N = 3, 3
    # uninterrupted
    W, ro = synth.make_tables(wl, DEV)
    tab = elf.Tables(W, ro)
    ws = workspace_for(wl, tab, range(K + N))
    bufs = core_buffers(wl)
    for i in range(K + N):
        core_step(wl, tab, ws, i, *bufs)
    torch.cuda.synchronize()
    ref_W, ref_out = W.clone(), [b.clone() for b in bufs]
    del W, ro, tab, ws, bufs
    # K steps, save, drop everything
    W, ro = synth.make_tables(wl, DEV)
    tab = elf.Tables(W, ro)
    ws = workspace_for(wl, tab, range(K))
    bufs = core_buffers(wl)
    for i in range(K):
        core_step(wl, tab, ws, i, *bufs)
    torch.cuda.synchronize()
    path = tmp_path / "tables.pt"
    torch.save({"tables": W.cpu(), "row_offset": ro.cpu(), "step": K}, path)
    del W, ro, tab, ws, bufs
    torch.cuda.empty_cache()
    # reload into new buffers and continue
    ck = torch.load(path, weights_only=True)
    W, ro = ck["tables"].to(DEV), ck["row_offset"].to(DEV)
    tab = elf.Tables(W, ro)
    ws = workspace_for(wl, tab, range(ck["step"], K + N))
    bufs = core_buffers(wl)
    for i in range(ck["step"], K + N):
        core_step(wl, tab, ws, i, *bufs)
    torch.cuda.synchronize()
    assert torch.equal(bits(W), bits(ref_W)), "tables differ after resuming"
    for got, ref, name in zip(bufs, ref_out, ("out", "emb", "dx0", "demb")):
        assert torch.equal(bits(got), bits(ref)), f"last step's {name} differs after resuming"
    # and the run did change the tables (the comparison is not between two untouched copies)
    W0, _ = synth.make_tables(wl, DEV)
    assert not torch.equal(bits(W0), bits(ref_W))


def dlrm_workload():
    return synth.WORKLOADS["train_step"].scaled(name="ckpt-dlrm", batch=517, rows=(3000, 50, 1234, 777),
                                                dim=32, bottom_mlp=(13, 64, 32))


def dlrm_model(wl):
    W, ro = synth.make_tables(wl, DEV)
    tab = elf.Tables(W, ro)
    step = dlrm.DLRMStep(wl, tab, DEV, top=(64, 32, 1))
    return W, tab, step


def dlrm_run(wl, tab, step, steps):
    for i in steps:
        idx, off = synth.make_indices(wl, DEV, batch_id=i)
        bags = elf.Bags(idx, off, wl.batch)
        ws = elf.alloc_workspace(tab, bags)
        step.train_step(synth.make_dense(wl, DEV, i), bags, synth.make_labels(wl, DEV, i), ws)


def test_whole_model_step_resumes_bitwise_from_a_checkpoint(tmp_path):
    wl = dlrm_workload()
    K, N = 2, 2
    W, tab, step = dlrm_model(wl)
    dlrm_run(wl, tab, step, range(K + N))
    torch.cuda.synchronize()
    ref = [W.clone(), step.bottom.master.clone(), step.bottom.copy.clone(), step.top.master.clone(),
           step.top.copy.clone(), step.loss.clone()]
    del W, tab, step
    W, tab, step = dlrm_model(wl)
    dlrm_run(wl, tab, step, range(K))
    torch.cuda.synchronize()
    path = tmp_path / "model.pt"
    torch.save({"tables": W.cpu(), "bottom_master": step.bottom.master.cpu(), "bottom_copy": step.bottom.copy.cpu(),
                "top_master": step.top.master.cpu(), "top_copy": step.top.copy.cpu(), "step": K}, path)
    del W, tab, step
    torch.cuda.empty_cache()
    ck = torch.load(path, weights_only=True)
    W, tab, step = dlrm_model(wl)  # fresh buffers at their initial values, then the saved state
    W.copy_(ck["tables"].to(DEV))
    step.bottom.master.copy_(ck["bottom_master"].to(DEV))
    step.bottom.copy.copy_(ck["bottom_copy"].to(DEV))
    step.top.master.copy_(ck["top_master"].to(DEV))
    step.top.copy.copy_(ck["top_copy"].to(DEV))
    dlrm_run(wl, tab, step, range(ck["step"], K + N))
    torch.cuda.synchronize()
    got = [W, step.bottom.master, step.bottom.copy, step.top.master, step.top.copy, step.loss]
    for g, r, name in zip(got, ref, ("tables", "bottom master", "bottom copy", "top master", "top copy", "loss")):
        assert torch.equal(bits(g), bits(r)), f"{name} differs after resuming"
