"""A whole training step captured in a HIP graph (both streams) replays to the same bits as
the eager calls, replay after replay, with eager work and synchronisations in between (GPU).

The step is the benchmark's: emb_dot_fwd storing the pooled vectors, the sort of the
lookups (emb_grad_prepare) on a side stream, dot_interact_bwd, then emb_grad_apply once the
sort is done.  The sort forks either after the forward or at the start of the step.
"""
import pytest
import torch

import embedding_lookup_feature_amd as elf
from embedding_lookup_feature_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


class Step:
    def __init__(self, W, ro, batches, wl, sort_from_start):
        B, F, D = wl.batch, wl.num_tables, wl.dim
        self.wl, self.tab, self.batches = wl, elf.Tables(W, ro), batches
        self.sort_from_start = sort_from_start
        self.emb = torch.empty((B, F, D), dtype=torch.bfloat16, device=DEV)
        self.out = torch.empty((B, wl.out_stride), dtype=torch.bfloat16, device=DEV)
        self.dx0 = torch.empty((B, D), dtype=torch.bfloat16, device=DEV)
        self.demb = torch.empty((B, F, D), dtype=torch.bfloat16, device=DEV)
        self.ws = elf.alloc_workspace(self.tab, batches[0][0])
        self.side = torch.cuda.Stream()
        self.fork, self.fwd_done, self.prepared = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()

    def __call__(self, i):
        bags, x0, G = self.batches[i % len(self.batches)]
        cur = torch.cuda.current_stream()
        if self.sort_from_start:
            self.fork.record(cur)
            self.side.wait_event(self.fork)
            elf.emb_grad_prepare(self.tab, bags, self.ws, stream=self.side)
            self.prepared.record(self.side)
        elf.emb_dot_fwd(self.tab, bags, x0, self.out, self.emb)
        if not self.sort_from_start:
            self.fwd_done.record(cur)
            self.side.wait_event(self.fwd_done)
            elf.emb_grad_prepare(self.tab, bags, self.ws, stream=self.side)
            self.prepared.record(self.side)
        elf.dot_interact_bwd(x0, self.emb, G, self.dx0, self.demb)
        cur.wait_event(self.prepared)
        elf.emb_grad_apply(self.tab, bags, self.demb, self.wl.lr, self.ws)


def bits(t):
    return t.view(torch.uint8).clone()


@pytest.mark.parametrize("sort_from_start", [False, True], ids=["sort-after-forward", "sort-from-start"])
def test_graph_replays_match_eager_steps(sort_from_start):
    wl = synth.WORKLOADS["train_step"].scaled(name="graph", batch=4096, rows=(5000,) * 26)
    W, ro = synth.make_tables(wl, DEV)
    batches = []
    for i in range(2):
        idx, off = synth.make_indices(wl, DEV, batch_id=i)
        batches.append((elf.Bags(idx, off, wl.batch), synth.make_x0(wl, DEV, i), synth.make_dout(wl, DEV, i)))
    order = [0, 1, 0, 0, 1]

    # eager chain
    eager = Step(W.clone(), ro, batches, wl, sort_from_start)
    ref = []
    for i in order:
        eager(i)
        torch.cuda.synchronize()
        ref.append((bits(eager.tab.weight), bits(eager.out), bits(eager.dx0), bits(eager.demb)))

    # graph chain: one graph per batch, captured without running, replayed in the same order
    graph = Step(W.clone(), ro, batches, wl, sort_from_start)
    gs = []
    for i in range(len(batches)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            graph(i)
        gs.append(g)
    torch.cuda.synchronize()
    assert torch.equal(bits(graph.tab.weight), bits(W)), "capture ran the step"
    noise = torch.randn(1 << 20, device=DEV)
    for n, i in enumerate(order):
        gs[i].replay()
        torch.cuda.synchronize()
        w, o, d, e = ref[n]
        assert torch.equal(bits(graph.tab.weight), w), f"replay {n}: tables differ"
        assert torch.equal(bits(graph.out), o), f"replay {n}: interaction output differs"
        assert torch.equal(bits(graph.dx0), d), f"replay {n}: dx0 differs"
        assert torch.equal(bits(graph.demb), e), f"replay {n}: demb differs"
        noise.mul_(1.0001).sum().item()  # the program's own eager work and a synchronisation
