"""Throughput of the embedding-bag + dot-interaction training step on one MI355X.

One step = the whole hot path over one batch of synthetic input already resident in HBM:
  emb_dot_fwd (the gather + the interaction forward, pooled vectors stored) ->
  dot_interact_bwd -> emb_grad_apply, with emb_grad_prepare (the sort of the lookups, which
  needs only the indices) on a side stream from the end of the forward, overlapping the
  backward
on the train_step workload (B = 65536, 26 fp32 tables x 100,000 x 128, bf16 activations,
Zipf(1.05) hotness-1 indices, SGD lr 0.01).  Eight distinct index batches rotate across
steps so that no step replays the previous one's rows from cache.

Prints one JSON line: samples/s, the step time, per-call HIP-event times (mean, median,
p10, p90) with algorithmic GB/s, the roofline of the dominant kernel (algorithmic bytes /
its average HIP-event time vs the 8 TB/s HBM peak, and vs the measured bandwidth of a
plain 4 GiB device copy), and the CPU oracle timed on a bounded sample of the same
workload.  --workload picks another configuration; forward-only ones time the fused
emb_dot_fwd (no pooled vectors stored), or the two forward calls with --separate-fwd.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {
    "k_emb_bag_fwd": ["include/embcore.h", "embedding_lookup_feature_amd/csrc/el_internal.hpp",
                      "embedding_lookup_feature_amd/csrc/emb_bag_fwd.hip"],
    "k_dot_fwd_mfma": ["include/embcore.h", "embedding_lookup_feature_amd/csrc/el_internal.hpp",
                       "embedding_lookup_feature_amd/csrc/el_mfma.hpp",
                       "embedding_lookup_feature_amd/csrc/dot_interact.hip"],
    "k_dot_bwd_mfma": ["include/embcore.h", "embedding_lookup_feature_amd/csrc/el_internal.hpp",
                       "embedding_lookup_feature_amd/csrc/el_mfma.hpp",
                       "embedding_lookup_feature_amd/csrc/dot_interact.hip"],
    "k_emb_dot_fwd": ["include/embcore.h", "embedding_lookup_feature_amd/csrc/el_internal.hpp",
                      "embedding_lookup_feature_amd/csrc/el_mfma.hpp",
                      "embedding_lookup_feature_amd/csrc/emb_dot_fwd.hip"],
}
KERNEL_SOURCES["k_emb_bag_long"] = KERNEL_SOURCES["k_emb_bag_fwd"]
KERNEL_SOURCES["k_dot_fwd_valu"] = KERNEL_SOURCES["k_dot_fwd_mfma"]
KERNEL_SOURCES["k_dot_fwd_wide"] = KERNEL_SOURCES["k_dot_fwd_mfma"]
KERNEL_SOURCES["k_dot_bwd_valu"] = KERNEL_SOURCES["k_dot_bwd_mfma"]
for _k, _f in (("k_seg_reduce", "grad_update.hip"), ("k_seg_fixup", "grad_update.hip"),
               ("k_build_vals", "grad_sort.hip"), ("k_sort_tiles", "grad_sort.hip"),
               ("k_tile_info", "grad_sort.hip"), ("k_radix_hist", "grad_sort.hip"),
               ("k_radix_scatter", "grad_sort.hip"), ("k_digit_scan", "grad_sort.hip")):
    KERNEL_SOURCES[_k] = ["include/embcore.h", "embedding_lookup_feature_amd/csrc/el_internal.hpp",
                          "embedding_lookup_feature_amd/csrc/" + _f]
KERNEL_OF_CALL = {"emb_bag_fwd": "k_emb_bag_fwd", "dot_interact_fwd": "k_dot_fwd_mfma",
                  "dot_interact_bwd": "k_dot_bwd_mfma", "emb_dot_fwd": "k_emb_dot_fwd",
                  "emb_dot_bwd": "k_dot_bwd_mfma"}


def kernel_of(call, wl):
    """The kernel a one-kernel call runs for this workload's shape: the interaction takes
    MFMA for 16-bit activations with D % 16 == 0 (the backward also D >= 32 and 16-byte
    gradient rows), the fp32 FMA kernels otherwise."""
    V, D = wl.num_tables + 1, wl.dim
    mfma = wl.act_dtype in ("bf16", "f16") and D % 16 == 0 and V <= 128
    row_bytes = D * (4 if wl.table_dtype == "f32" else 2)
    if call == "emb_bag_fwd" and wl.bag[0] == "poisson" and wl.bag[1] >= 4 and row_bytes >= 128:
        return "k_emb_bag_long"  # long bags: one bag per lane group
    if call == "dot_interact_fwd" and not mfma:
        return "k_dot_fwd_valu"
    if call == "dot_interact_fwd" and V > 32:  # several 32-row tiles: four wavefronts per sample
        return "k_dot_fwd_wide"
    if call == "dot_interact_bwd" and not (mfma and D >= 32 and wl.out_stride % 8 == 0):
        return "k_dot_bwd_valu"
    return KERNEL_OF_CALL[call]


def fused_bwd_ok(wl):
    """The shapes emb_dot_bwd's fused kernel covers (include/embcore.h)."""
    V, D = wl.num_tables + 1, wl.dim
    return (wl.act_dtype in ("bf16", "f16") and D % 16 == 0 and D >= 32 and V <= 32
            and (V + 31) // 32 * 16 * (D // 8) <= 256 and wl.out_stride % 8 == 0)


def fused_fwd_ok(wl):
    """The shapes emb_dot_fwd's fused kernel (no pooled-vector output) covers
    (include/embcore.h): 16-bit activations, D % 16 == 0, at most 64 tables."""
    return wl.act_dtype in ("bf16", "f16") and wl.dim % 16 == 0 and wl.num_tables <= 64


def metric_name(wl):
    what = "fwd+bwd" if wl.backward else "fwd"
    return f"samples/s {what} (emb-bag + dot interaction) at batch {wl.batch}; achieved HBM GB/s"


def algorithmic_bytes(wl, nnz, store_emb=None):
    """Bytes each call must move at minimum (every lookup's row counted; caches may serve
    part of them), per launch.  store_emb: the training forward stores the pooled vectors
    (default: whenever the workload has a backward)."""
    if store_emb is None:
        store_emb = wl.backward
    B, F, D = wl.batch, wl.num_tables, wl.dim
    st = 4 if wl.table_dtype == "f32" else 2
    sa = 4 if wl.act_dtype == "f32" else 2
    S = wl.out_stride
    V = F + 1
    return {
        # rows + indices + offsets + pooled output
        "emb_bag_fwd": nnz * D * st + 4 * nnz + 4 * (F * B + 1) + B * F * D * sa,
        # x0 + emb in, interaction rows out
        "dot_interact_fwd": B * V * D * sa + B * S * sa,
        # rows + indices + offsets + x0 in, interaction rows out (+ pooled vectors out when
        # the backward needs them); the pooled vectors are not read back from HBM
        "emb_dot_fwd": nnz * D * st + 4 * nnz + 4 * (F * B + 1) + B * D * sa + B * S * sa
                       + (B * F * D * sa if store_emb else 0),
        # dout in, x0 + emb in, dx0 + demb out
        "dot_interact_bwd": B * S * sa + 2 * B * V * D * sa,
        # dout + x0 + rows + indices + offsets in, dx0 + demb out
        "emb_dot_bwd": B * S * sa + B * D * sa + nnz * D * st + 4 * nnz + 4 * (F * B + 1)
                       + B * V * D * sa,
        # keys + bag ids read once, gradients gathered once, touched rows read + written (the
        # sort's own passes are not counted)
        "emb_grad_reduce_update": None,  # filled in by the caller (needs the unique-row count)
    }


def sort_passes(wl):
    """Radix passes of the gradient sort: 8-bit digits over the local rows of the largest
    table (every table's lookups are sorted in place by local row)."""
    key_bits = max(1, int(max(wl.rows) - 1).bit_length())
    return (key_bits + 7) // 8


def sort_start(wl, nnz):
    """Where the sort of the lookups starts on its side stream: it needs only the indices, so
    it may run beside the forward too, but the gather's row reuse in L2 suffers from it; it
    starts with the step only when its passes (keys + bag ids read and written per 8-bit
    digit) move more bytes than the interaction backward it would otherwise hide behind."""
    sa = 4 if wl.act_dtype == "f32" else 2
    sort_bytes = 16 * nnz * sort_passes(wl)
    bwd_bytes = wl.batch * wl.out_stride * sa + 2 * wl.batch * (wl.num_tables + 1) * wl.dim * sa
    return "fwd" if sort_bytes > bwd_bytes else "bwd"


def source_digest(paths):
    """sha256 over the code of the given files (repo-relative), in order: C/C++ comments
    removed and whitespace runs folded, so that an edit of comments alone keeps the digest."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` (or the sum over the kernels of a call, joined by
    " + ") from the committed rocprofv3 counter summary, or None when there is none for this
    workload or a kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        entries = json.load(f)
    total = 0
    for k in kernel.split(" + "):
        hit = [e for e in entries.get("kernels", []) if e["workload"] == workload and e["kernel"] == k]
        if not hit or source_digest(hit[0]["sources"]) != hit[0]["sources_sha256"]:
            return None
        total += hit[0]["bytes_per_launch"]
    return total


def distinct_twin(wl):
    """Name of the catalogued distinct-row workload with `wl`'s shapes and dtypes, or None."""
    from embedding_lookup_feature_amd import synth
    for name, w in synth.WORKLOADS.items():
        if w.index_dist == "distinct" and (w.batch, tuple(w.rows), w.dim, w.table_dtype, w.act_dtype, w.bag) == \
                (wl.batch, tuple(wl.rows), wl.dim, wl.table_dtype, wl.act_dtype, wl.bag):
            return name
    return None


def hbm_calibration(dev, gib=4, reps=5):
    """GB/s that the library's HBM calibration kernels reach on this GPU: k_copy_calib over
    `gib` GiB of traffic each (read only, write only, copy, and a 3:1 read/write mix), and
    k_gather_calib reading distinct random rows of 128 / 256 / 512 bytes (half of a `gib` GiB
    table) and writing them contiguously (gather_*: reads + writes + indices), writing only
    their first half (gather_*_write_half: the mix of fp32 rows pooled into 16-bit outputs)
    or only reading them (gather_read_*).  Each figure is the median of `reps` launches timed with
    HIP events after one warm-up launch, and the best over the cache policies of the kernel's
    loads and stores (plain or non-temporal; `policy` records which won)."""
    import embedding_lookup_feature_amd as elf
    from embedding_lookup_feature_amd import embcore as ec
    n = gib << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device=dev)

    def median_ms(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    NL, NS = ec.EL_CALIB_NT_LOADS, ec.EL_CALIB_NT_STORES
    names = {0: "plain", NL: "nt loads", NS: "nt stores", NL | NS: "nt loads+stores"}
    res, policy = {}, {}

    def best(name, traffic, run, policies):
        ms = {p: median_ms(lambda: run(p)) for p in policies}
        p = min(ms, key=ms.get)
        res[name] = round(traffic / (ms[p] * 1e-3) / 1e9, 1)
        policy[name] = names[p]

    both = (0, NL, NS, NL | NS)
    for name, mode, pols in (("read", ec.EL_CALIB_READ, (0, NL)), ("write", ec.EL_CALIB_WRITE, (0, NS)),
                             ("copy", ec.EL_CALIB_COPY, both), ("read3_write1", ec.EL_CALIB_READ3_WRITE1, both)):
        best(name, n, lambda p: elf.hbm_calib(mode | p, a, b, n), pols)
    g = torch.Generator(device=dev)
    g.manual_seed(12345)
    for rb in (128, 256, 512):
        rows = n // rb
        nr = (n // 2) // rb  # distinct random rows, half the table's bytes, read once each
        idx = torch.randperm(rows, generator=g, device=dev)[:nr].to(torch.int32)
        best(f"gather_{rb}B", 2 * nr * rb + 4 * nr,
             lambda p: elf.hbm_calib(ec.EL_CALIB_GATHER | p, a, b, 0, idx=idx, row_bytes=rb), both)
        best(f"gather_read_{rb}B", nr * rb + 4 * nr,
             lambda p: elf.hbm_calib(ec.EL_CALIB_GATHER_READ | p, a, b, 0, idx=idx, row_bytes=rb), (0, NL))
        if rb >= 256:  # rows pooled into outputs of half their size (fp32 rows, 16-bit outputs)
            best(f"gather_{rb}B_write_half", nr * rb * 3 // 2 + 4 * nr,
                 lambda p: elf.hbm_calib(ec.EL_CALIB_GATHER | p, a, b, rb // 2, idx=idx, row_bytes=rb), both)
        del idx
    del a, b
    torch.cuda.empty_cache()
    res["policy"] = policy
    return res


# The calibrated ceiling each call is compared with: the streaming mix closest to its traffic.
# The gathers are read-mostly, and random rows of these sizes read as fast as a stream
# (gather_read_* ~ read), so theirs is the streaming read.
def ceiling_of(call, wl, calib):
    if not calib:
        return None, None
    if call in ("emb_bag_fwd", "emb_dot_fwd", "emb_dot_bwd", "emb_cat_fwd"):
        key = "read"
    elif call in ("emb_grad_reduce_update", "emb_grad_apply"):
        key = "read3_write1"
    else:  # interaction forward / backward: read and write about equally
        key = "copy"
    return key, calib.get(key)


def pct(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="train_step")
    ap.add_argument("--batches", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB once (a plain copy kernel "
                         "of known size, to scale HBM byte counters)")
    ap.add_argument("--separate-fwd", action="store_true",
                    help="time emb_bag_fwd + dot_interact_fwd instead of emb_dot_fwd (which, for "
                         "forward-only workloads, does not store the pooled vectors at all, and in "
                         "training runs the two kernels on cache-sized chunks of samples)")
    ap.add_argument("--overlap-sort", choices=["auto", "none", "fwd", "bwd", "next"], default="auto",
                    help="run the gradient sort (emb_grad_prepare) on a side stream, from the start of "
                         "the step (fwd) or from the end of the forward (bwd), then emb_grad_apply; "
                         "next: the sort of the next batch (it needs only that batch's indices) "
                         "starts beside this step's update, into the other of two workspaces; "
                         "auto: from the start when the sort's passes move more bytes than the "
                         "interaction backward, else from the end of the forward")
    ap.add_argument("--recompute-emb", action="store_true",
                    help="training: do not store the pooled vectors in the forward (emb_dot_fwd "
                         "without emb_out); rebuild them from the tables in the backward "
                         "(emb_dot_bwd) instead of reading them back in dot_interact_bwd")
    ap.add_argument("--inference-sweep", action="store_true",
                    help="forward-only latency / throughput over batch sizes 1 .. 1,048,576 on the "
                         "large fp16 tables (emb_dot_fwd, pooled vectors not stored); one JSON line "
                         "per batch size instead of the step line")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of HIP graphs, one per index batch, each capturing one whole "
                         "step (both streams); per-call times still come from eager calls")
    ap.add_argument("--hash-indices", action="store_true",
                    help="pass the floor-modulo index hashing flag to every call that reads the indices "
                         "(the generated indices are already in range, so results are unchanged; the "
                         "line then shows what the hashing costs)")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the HBM calibration kernels (4 GiB each) that measure the bandwidth "
                         "streaming kernels reach on this GPU")
    ap.add_argument("--no-uniform-control", action="store_true",
                    help="skip the no-reuse gather control (emb_bag_fwd on the workload's shapes "
                         "with every table's lookups distinct rows, so that no row comes from cache)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import embedding_lookup_feature_amd as elf
    from embedding_lookup_feature_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.inference_sweep:
        inference_sweep(dev, args.workload if args.workload != "train_step" else "large_table")
        return
    if args.workload == "dlrm_step":
        dlrm_bench(args, dev)
        return
    wl = synth.WORKLOADS[args.workload]
    B, F, D = wl.batch, wl.num_tables, wl.dim
    act = synth.act_dtype(wl)

    W, ro = synth.make_tables(wl, dev)
    tab = elf.Tables(W, ro)
    batches = []
    for i in range(args.batches):
        idx, off = synth.make_indices(wl, dev, batch_id=i)
        batches.append((elf.Bags(idx, off, B), synth.make_x0(wl, dev, i), synth.make_dout(wl, dev, i), idx, off))
    emb = torch.empty((B, F, D), dtype=act, device=dev)
    out = torch.empty((B, wl.out_stride), dtype=act, device=dev)
    if wl.backward:
        dx0 = torch.empty((B, D), dtype=act, device=dev)
        demb = torch.empty((B, F, D), dtype=act, device=dev)
        ws = torch.empty(max(elf.emb_grad_workspace_bytes(tab, b[0]) for b in batches),
                         dtype=torch.uint8, device=dev)

    if args.overlap_sort == "auto":
        args.overlap_sort = sort_start(wl, batches[0][3].numel()) if wl.backward else "none"
    if args.overlap_sort == "next" and args.graph:
        sys.exit("--overlap-sort next leaves the next batch's sort running past the step, which a "
                 "graph of one step cannot hold")
    overlap = wl.backward and args.overlap_sort != "none"
    nxt = overlap and args.overlap_sort == "next"
    # next: two workspaces, batch i's in wss[i % 2] (the sort of batch i + 1 writes the other
    # one while the update of batch i reads this one)
    wss = ([ws, torch.empty_like(ws)] if nxt else [ws, ws]) if wl.backward else None
    fused_fwd = not args.separate_fwd
    # training: store the pooled vectors and read them back (the faster order here), or
    # with --recompute-emb rebuild them in the backward where the fused backward covers
    # the shape
    recompute = wl.backward and fused_fwd and args.recompute_emb and fused_bwd_ok(wl)
    # forward-only shapes the fused kernel does not cover store the pooled vectors (chunked
    # gather + interaction)
    store_emb = (wl.backward and not recompute) or (fused_fwd and not fused_fwd_ok(wl))
    bwd_name = "emb_dot_bwd" if recompute else "dot_interact_bwd"
    fwd_names = ["emb_dot_fwd"] if fused_fwd else ["emb_bag_fwd", "dot_interact_fwd"]
    if not wl.backward:
        names = fwd_names
    elif overlap:
        names = fwd_names + [bwd_name, "emb_grad_apply"]
    else:
        names = fwd_names + [bwd_name, "emb_grad_reduce_update"]
    hx = args.hash_indices
    main_stream = torch.cuda.current_stream()
    side = torch.cuda.Stream() if overlap else None  # default priority
    prepared = [torch.cuda.Event(), torch.cuda.Event()]  # sort of batch i done: prepared[i % 2]
    fwd_done = torch.cuda.Event()
    fork = torch.cuda.Event()

    def start_sort(i, side_ev):
        # the workspace is free once the update that last read it is done: from the start of
        # the step, fork from the step's stream (the update ran there before); from the end of
        # the forward, the wait for the forward already implies it; next: the fork at the end
        # of this step's backward comes after the previous update, the other workspace's
        if args.overlap_sort in ("fwd", "next"):
            fork.record(torch.cuda.current_stream())
            side.wait_event(fork)
        if side_ev: side_ev[0].record(side)
        elf.emb_grad_prepare(tab, batches[i % len(batches)][0], wss[i % 2], hash_indices=hx, stream=side)
        if side_ev: side_ev[1].record(side)
        prepared[i % 2].record(side)

    def step(i, ev=None, side_ev=None, wait_ev=None):
        """One pass of the path over batch i.  With overlap, the sort of the lookups (it needs
        only the indices) runs on a side stream while the forward and the interaction
        backward run; the update waits for it."""
        bags, x0, G = batches[i % len(batches)][:3]
        if overlap and args.overlap_sort == "fwd":
            start_sort(i, side_ev)
        if ev: ev[0].record()
        k = 1
        if fused_fwd:  # pooled vectors stored only when the backward reads them back
            elf.emb_dot_fwd(tab, bags, x0, out, emb if store_emb else None, hash_indices=hx)
        else:
            elf.emb_bag_fwd(tab, bags, emb, hash_indices=hx)
            if ev: ev[k].record()
            k += 1
            elf.dot_interact_fwd(x0, emb, out)
        if ev: ev[k].record()
        k += 1
        if not wl.backward:
            return
        if overlap and args.overlap_sort == "bwd":
            fwd_done.record(torch.cuda.current_stream())
            side.wait_event(fwd_done)
            start_sort(i, side_ev)
        if recompute:
            elf.emb_dot_bwd(tab, bags, x0, G, dx0, demb, hash_indices=hx)
        else:
            elf.dot_interact_bwd(x0, emb, G, dx0, demb)
        if ev: ev[k].record()
        k += 1
        if overlap:
            if nxt:  # the next batch's sort, beside this update and what follows it
                start_sort(i + 1, side_ev)
            torch.cuda.current_stream().wait_event(prepared[i % 2])
            if wait_ev is not None:  # the update's own time starts once the sort is done
                wait_ev.record()
            elf.emb_grad_apply(tab, bags, demb, wl.lr, wss[i % 2], hash_indices=hx)
        else:
            elf.emb_grad_reduce_update(tab, bags, demb, wl.lr, ws, hash_indices=hx)
        if ev: ev[k].record()

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def prime():
        """next: the sort of the first step's batch, before the steps (each step sorts the
        batch after it, so a run of K steps still sorts K batches)."""
        if nxt:
            elf.emb_grad_prepare(tab, batches[0][0], wss[0], hash_indices=hx, stream=side)
            prepared[0].record(side)
            torch.cuda.synchronize()

    prime()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graphs = None
    if args.graph:
        # one graph per index batch, each one whole step; captured after the warm-up (which
        # filled the library's host-side occupancy cache), replayed in batch order
        graphs = []
        for i in range(len(batches)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(len(batches)):
            graphs[i].replay()
        torch.cuda.synchronize()

    # timed region: K whole steps, no per-call events (nothing but the path in the stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prime()
    torch.cuda.synchronize()
    t0.record()
    if side is not None:
        side.wait_stream(main_stream)  # no side-stream work starts before t0
    for i in range(args.steps):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step(i)
    if nxt:  # the sort of the batch after the last step is part of the K steps' work
        main_stream.wait_event(prepared[args.steps % 2])
    t1.record()  # the last update waited for the last sort, so all work is before t1
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # per-call durations: HIP events around each call (recorded on the stream the calls are
    # enqueued on, torch's current stream), over the same number of steps
    nev = len(names) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    wevs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    prime()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i], sevs[i] if overlap else None, wevs[i] if overlap else None)
    torch.cuda.synchronize()
    call_samples = {n: [e[k].elapsed_time(e[k + 1]) for e in evs] for k, n in enumerate(names)}
    if overlap:  # side stream: the sort, overlapping the calls above
        call_samples["emb_grad_prepare"] = [e[0].elapsed_time(e[1]) for e in sevs]
        if "emb_grad_apply" in names:  # from the end of the wait for the sort
            ka = names.index("emb_grad_apply")
            call_samples["wait_for_sort"] = [e[ka].elapsed_time(w) for e, w in zip(evs, wevs)]
            call_samples["emb_grad_apply"] = [w.elapsed_time(e[ka + 1]) for e, w in zip(evs, wevs)]
    call_ms = {n: float(np.mean(v)) for n, v in call_samples.items()}
    # the sort alone (nothing beside it), on the batches of the timed steps: what the side
    # stream's figure above would be without the calls it overlaps
    sort_alone = None
    if overlap:
        ea = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        torch.cuda.synchronize()
        for i, (e0, e1) in enumerate(ea):
            e0.record()
            elf.emb_grad_prepare(tab, batches[i % len(batches)][0], ws, hash_indices=hx)
            e1.record()
            torch.cuda.synchronize()
        sort_alone = float(np.median([a.elapsed_time(b) for a, b in ea]))

    # the gather with no row reuse: emb_bag_fwd alone on the same shapes with every table's
    # lookups distinct rows (each row read once, so its algorithmic bytes all come from HBM)
    uniform = None
    if not args.no_uniform_control and wl.bag == ("one",) and wl.index_dist == "zipf" \
            and max(wl.batch, 1) <= min(wl.rows):
        wu = wl.scaled(name=wl.name + "_distinct_control", index_dist="distinct")
        iu, ou = synth.make_indices(wu, dev)
        bu = elf.Bags(iu, ou, B)
        eu = torch.empty((B, F, D), dtype=act, device=dev)
        for _ in range(3):
            elf.emb_bag_fwd(tab, bu, eu)
        torch.cuda.synchronize()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for e0, e1 in es:
            e0.record()
            elf.emb_bag_fwd(tab, bu, eu)
            e1.record()
        torch.cuda.synchronize()
        uniform = float(np.mean([a.elapsed_time(b) for a, b in es]))
        del iu, ou, bu, eu
        torch.cuda.empty_cache()

    calib = None if args.no_calib else hbm_calibration(dev)

    nnz = batches[0][3].numel()
    algo = algorithmic_bytes(wl, nnz, store_emb)
    idx0, off0 = batches[0][3], batches[0][4]
    # unique rows touched (for the update's row read + write), from the input indices
    keys = idx0.long() + torch.repeat_interleave(ro[:-1], (off0[1:].long() - off0[:-1].long()).view(F, B).sum(1))
    U = int(torch.unique(keys).numel())
    st = 4 if wl.table_dtype == "f32" else 2
    sa = 4 if wl.act_dtype == "f32" else 2
    algo["emb_grad_reduce_update"] = 8 * nnz + nnz * D * sa + 2 * U * D * st
    algo["emb_grad_apply"] = algo["emb_grad_reduce_update"]
    # the sort: keys + bag ids read and written once per 8-bit radix pass over local rows
    algo["emb_grad_prepare"] = 16 * nnz * sort_passes(wl)
    timed = [n for n in call_samples if n != "wait_for_sort"]
    algo = {n: algo[n] for n in timed}
    calls = {}
    for n in timed:
        v = call_samples[n]
        c = {"ms": round(call_ms[n], 4), "median_ms": round(pct(v, 50), 4),
             "p10_ms": round(pct(v, 10), 4), "p90_ms": round(pct(v, 90), 4),
             "algo_bytes": int(algo[n]), "algo_gbps": round(algo[n] / (call_ms[n] * 1e-3) / 1e9, 1)}
        ck, cg = ceiling_of(n, wl, calib)
        if cg:
            c["ceiling"] = ck
            c["frac_of_ceiling"] = round(c["algo_gbps"] / cg, 4)
        if n == "emb_grad_prepare":
            c["stream"] = "side (overlaps " + ("the forward and " if args.overlap_sort == "fwd" else "") + \
                          "the interaction backward)"
            if sort_alone is not None:
                c["alone_median_ms"] = round(sort_alone, 4)
        calls[n] = c
    if "wait_for_sort" in call_samples:
        v = call_samples["wait_for_sort"]
        calls["wait_for_sort"] = {"ms": round(float(np.mean(v)), 4), "median_ms": round(pct(v, 50), 4),
                                  "note": "main stream idle between the interaction backward and "
                                          "emb_grad_apply, waiting for the side-stream sort"}
    step_bytes = sum(algo[n] for n in names)  # the sort's passes are not counted
    # dominant kernel: the longest of the one-kernel calls (the update call is a sequence of
    # short sort / reduce kernels, each well below the interaction kernels; in training
    # emb_dot_fwd is a sequence of gather and interaction launches)
    single = [n for n in names if n in KERNEL_OF_CALL and not (n == "emb_dot_fwd" and store_emb)]
    if single:
        dom = max(single, key=lambda n: call_ms[n])
        kernel = kernel_of(dom, wl)
    else:  # a forward-only line whose one call runs the gather and the interaction in chunks
        dom, kernel = names[0], kernel_of("emb_bag_fwd", wl) + " + " + kernel_of("dot_interact_fwd", wl)
    def roofline_of(call, kernel, ms, nbytes, note=None, traffic_workload=None):
        a = nbytes / (ms * 1e-3) / 1e9
        r = {"bound": "hbm", "kernel": kernel, "call": call, "achieved": round(a, 1), "peak": HBM_PEAK_GBPS,
             "unit": "GB/s", "frac": round(a / HBM_PEAK_GBPS, 4),
             "traffic": measured_traffic(traffic_workload or wl.name, kernel)}
        ck, cg = ceiling_of(call, wl, calib)
        if cg:
            r.update({"ceiling": ck, "ceiling_gbps": cg, "frac_of_ceiling": round(a / cg, 4)})
        if r["traffic"] is not None:  # the HBM rate by the counters' bytes
            tg = r["traffic"] / (ms * 1e-3) / 1e9
            r.update({"traffic_gbps": round(tg, 1), "traffic_frac": round(tg / HBM_PEAK_GBPS, 4)})
        if a > HBM_PEAK_GBPS:
            reuse = ("the algorithmic bytes count every lookup's rows, and caches serve the rows that "
                     "lookups share, so they exceed what HBM alone could deliver in this time")
            note = f"{note}; {reuse}" if note else reuse
        if note:
            r["note"] = note
        return r

    roofline = roofline_of(dom, kernel, call_ms[dom], algo[dom])
    rooflines = [roofline]
    upd = "emb_grad_apply" if "emb_grad_apply" in call_ms else (
        "emb_grad_reduce_update" if "emb_grad_reduce_update" in call_ms else None)
    if upd:
        rooflines.append(roofline_of(upd, "k_seg_reduce + k_seg_fixup", call_ms[upd], algo[upd],
                                     "the update's kernels in sequence; HIP-event time of the call"))
    if uniform is not None:
        gb = algorithmic_bytes(wl, nnz)["emb_bag_fwd"]
        rooflines.append(roofline_of("emb_bag_fwd", "k_emb_bag_fwd", uniform, gb,
                                     "control on the workload's shapes with every table's lookups distinct "
                                     "rows (no row reuse), mean of 20 HIP-event timed calls; traffic from the "
                                     "counters of the distinct-row workload of the same shapes (another seed "
                                     "of the same draw)", traffic_workload=distinct_twin(wl)))

    sort_where = {"fwd": "from the start of the step", "bwd": "from the end of the forward",
                  "next": "for the next batch, beside this step's update"}.get(args.overlap_sort)
    result = {
        "metric": metric_name(wl),
        "value": round(B / (ms_per_step * 1e-3), 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.act_dtype == "bf16" else wl.act_dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.description}", "global_batch": B,
                   "tables": F, "rows_per_table": wl.rows[0] if len(set(wl.rows)) == 1 else "varied",
                   "total_rows": wl.total_rows, "dim": D,
                   "table_dtype": wl.table_dtype, "act_dtype": wl.act_dtype, "nnz": int(nnz),
                   "unique_rows": U, "parallelism": "single-gpu",
                   "launch": "HIP graph replay, one graph per step" if args.graph else "eager",
                   "calls": " -> ".join(names) + (f" (emb_grad_prepare on a side stream {sort_where})"
                                                  if overlap else ""),
                   "hash_indices": bool(hx)},
        "hbm_gbps_algorithmic": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "calls": calls,
        "roofline": roofline,
        "rooflines": rooflines,
    }
    if calib:
        result["hbm_calibration_gbps"] = calib
    if not args.no_cpu_baseline:
        result["cpu_baseline"], omp = cpu_baseline(wl, W, ro, batches[0], args.cpu_seconds)
        if omp:
            result["cpu_baseline_openmp"] = omp
    print(json.dumps(result), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def dlrm_bench(args, dev):
    """The whole DLRM training step on the train_step shapes: bottom MLP 13-512-256-128,
    emb-bag + dot interaction, top MLP 479-1024-1024-512-256-1 (its input zero-padded to 512
    columns), logistic loss, backward of
    every stage, SGD (lr 0.01) on the dense parameters and the embedding rows; the sort of
    the lookups on a side stream from the start of the step.  Reports samples/s, per-stage
    HIP-event times, and each dense layer's forward / backward timed on its own (TFLOP/s vs
    the bf16 MFMA peak); the roofline object is the dominant dense-layer product."""
    import embedding_lookup_feature_amd as elf
    from embedding_lookup_feature_amd import dlrm, synth

    wl = synth.WORKLOADS["train_step"]
    B = wl.batch
    W, ro = synth.make_tables(wl, dev)
    tab = elf.Tables(W, ro)
    batches = []
    for i in range(args.batches):
        idx, off = synth.make_indices(wl, dev, batch_id=i)
        batches.append((elf.Bags(idx, off, B), synth.make_dense(wl, dev, i), synth.make_labels(wl, dev, i)))
    step = dlrm.DLRMStep(wl, tab, dev)
    ws = torch.empty(max(elf.emb_grad_workspace_bytes(tab, b[0]) for b in batches), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()  # default priority

    def run(i, mark=None):
        bags, dense, labels = batches[i % len(batches)]
        step.train_step(dense, bags, labels, ws, side=side, mark=mark)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    side.wait_stream(torch.cuda.current_stream())
    for i in range(args.steps):
        run(i)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # per-stage HIP events on the main stream (the sort runs beside them on the side stream)
    stage = {}
    for i in range(args.steps):
        marks = [("start", torch.cuda.Event(enable_timing=True))]
        marks[0][1].record()

        def mark(name, marks=marks):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append((name, e))
        run(i, mark)
        torch.cuda.synchronize()
        for (_, a), (n, b) in zip(marks[:-1], marks[1:]):
            stage.setdefault(n, []).append(a.elapsed_time(b))
    stages = {n: {"median_ms": round(pct(v, 50), 4), "p10_ms": round(pct(v, 10), 4),
                  "p90_ms": round(pct(v, 90), 4)} for n, v in stage.items()}

    # each dense layer on its own: forward, and backward (data + weight gradients)
    layers = []
    reps = max(10, args.steps // 5)
    shapes = [("bottom", i, s) for i, s in enumerate(step.bottom.shapes)] + \
             [("top", i, s) for i, s in enumerate(step.top.shapes)]
    real_k = dict(zip(range(len(shapes)), [wl.bottom_mlp[0]] + [k for (_, k) in step.bottom.shapes[1:]] +
                      [wl.out_width] + [k for (_, k) in step.top.shapes[1:]]))
    for li, (which, i, (N, K)) in enumerate(shapes):
        mlp = step.bottom if which == "bottom" else step.top
        acts = step.h_bot if which == "bottom" else step.h_top
        x = (batches[0][1] if i == 0 else acts[i - 1]) if which == "bottom" else (step.inter if i == 0 else acts[i - 1])
        y = acts[i]
        relu = which == "bottom" or i < len(mlp.w) - 1
        dz = torch.zeros_like(y)
        dx = torch.empty_like(x) if not (which == "bottom" and i == 0) else None
        res = {}
        for kind in ("fwd", "bwd"):
            es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for e0, e1 in es:
                e0.record()
                if kind == "fwd":
                    elf.linear_fwd(x, mlp.w[i], mlp.b[i], y, relu=relu)
                else:
                    elf.linear_bwd(x, mlp.w[i], dz, mlp.dw[i], mlp.db[i], dx=dx, relu_mask=dx is not None and i > 0,
                                   workspace=step.lin_ws)
                e1.record()
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in es]))
            flops = 2 * B * N * real_k[li] * (1 if kind == "fwd" else (2 if dx is not None else 1))
            res[kind] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        layers.append({"layer": f"{which}{i}", "K": real_k[li], "N": N, **res})
    dom = max(layers, key=lambda l: l["fwd"]["ms"] + l["bwd"]["ms"])
    achieved = dom["fwd"]["tflops"]
    flops = step.dense_flops()
    total_dense = sum(flops.values())
    dense_ms = sum(l["fwd"]["ms"] + l["bwd"]["ms"] for l in layers)
    result = {
        "metric": f"samples/s fwd+bwd, whole DLRM step (bottom MLP + emb-bag + dot interaction + top MLP "
                  f"+ logistic loss, SGD) at batch {B}",
        "value": round(B / (ms_per_step * 1e-3), 1),
        "unit": "samples/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dlrm_step: train_step shapes (26 fp32 tables x 100,000 x 128, Zipf(1.05) "
                               "hotness 1) + bottom MLP 13-512-256-128 + top MLP 479-1024-1024-512-256-1 "
                               "+ logistic loss on Bernoulli(0.25) labels, SGD lr 0.01 everywhere",
                   "global_batch": B, "parallelism": "single-gpu"},
        "dense_gflop_per_step": round(total_dense / 1e9, 1),
        "dense_tflops_in_isolation": round(total_dense / (dense_ms * 1e-3) / 1e12, 1),
        "stages": stages,
        "dense_layers": layers,
        "roofline": {"bound": "mfma", "kernel": f"k_gemm forward, {dom['layer']} ({dom['K']} -> {dom['N']})",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = dlrm_cpu_baseline(wl, W, ro, step, batches[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


def dlrm_cpu_baseline(wl, W, ro, step, batch, seconds):
    """The oracle's whole DLRM step (forward, loss, backward, SGD of the dense layers and of
    the touched embedding rows) over the first n samples of batch 0, single-threaded and
    pinned to one core; n sized for about `seconds`."""
    from oracle import oracle as orc
    from tests.helpers import sub_batch, to_np

    bags, dense, labels = batch
    F, B, D, dt = wl.num_tables, wl.batch, wl.dim, wl.act_dtype
    W_h, ro_h = to_np(W), to_np(ro)
    idx_h, off_h = to_np(bags.indices), to_np(bags.offsets)
    dense_h, lab_h = to_np(dense), to_np(labels)
    bw = [to_np(w) for w in step.bottom.w]
    bb = [to_np(b) for b in step.bottom.b]
    tw = [to_np(w) for w in step.top.w]
    tb = [to_np(b) for b in step.top.b]
    bm, tm = to_np(step.bottom.master), to_np(step.top.master)

    def run(n):
        si, so, nb = sub_batch(idx_h, off_h, F, B, np.arange(n))
        t = time.perf_counter()
        hs = [dense_h[:n]]
        for w, b in zip(bw, bb):
            hs.append(orc.linear_fwd(hs[-1], dt, w, dt, b, True, dt))
        emb = orc.emb_bag_fwd(W_h, wl.table_dtype, ro_h, si, so, nb, D, dt)
        ts = [orc.dot_interact_fwd(hs[-1], emb, dt, dt, step.inter.shape[1])]
        for j, (w, b) in enumerate(zip(tw, tb)):
            ts.append(orc.linear_fwd(ts[-1], dt, w, dt, b, j < len(tw) - 1, dt))
        _, dz = orc.bce_logits(ts[-1], dt, lab_h[:n], dt)
        dz = dz.reshape(n, 1)
        for j in reversed(range(len(tw))):
            dz, _, _ = orc.linear_bwd(ts[j], dt, tw[j], dt, dz, dt, dx_dtype=dt, relu_mask=j > 0)
        dx0, demb = orc.dot_interact_bwd(hs[-1], emb, dt, dz, dt, dt)
        dz = orc.relu_bwd(dx0, hs[-1], dt)
        for j in reversed(range(len(bw))):
            dz, _, _ = orc.linear_bwd(hs[j], dt, bw[j], dt, dz, dt, dx_dtype=dt if j > 0 else None,
                                      relu_mask=j > 0)
        orc.sgd_dense(bm, np.zeros_like(bm), wl.lr)
        orc.sgd_dense(tm, np.zeros_like(tm), wl.lr)
        orc.grad_reduce_update(W_h, wl.table_dtype, ro_h, si, so, nb, demb, dt, wl.lr)
        return time.perf_counter() - t

    model, nproc = cpu_info()
    old = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(old)})
    try:
        probe = 16
        dt_probe = run(probe)
        n = int(min(B, max(probe, probe * seconds / max(dt_probe, 1e-6))))
        dt_run = run(n)
    finally:
        os.sched_setaffinity(0, old)
    return {"value": round(n / dt_run, 1), "unit": "samples/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {B} samples of batch 0: the whole step (dense layers, full tables, "
                      f"SGD of all dense parameters and a full-table copy for the row update), "
                      f"single-threaded C oracle pinned to one core, {dt_run:.1f} s",
            "host_cpu": model, "host_cpus_visible": nproc}


def inference_sweep(dev, workload, sizes=(1, 16, 64, 256, 4096, 65536, 262144, 1048576), iters=100):
    """Forward-only serving figure: for each batch size, `iters` single calls of emb_dot_fwd
    (gather + interaction, pooled vectors kept on chip), each timed with its own HIP events;
    latency percentiles and samples/s = B / mean latency.  Two index batches alternate."""
    import embedding_lookup_feature_amd as elf
    from embedding_lookup_feature_amd import synth
    base = synth.WORKLOADS[workload]
    W, ro = synth.make_tables(base, dev)
    tab = elf.Tables(W, ro)
    for B in sizes:
        wl = base.scaled(batch=B)
        batches = []
        for i in range(2):
            idx, off = synth.make_indices(wl, dev, batch_id=i)
            batches.append((elf.Bags(idx, off, B), synth.make_x0(wl, dev, i)))
        out = torch.empty((B, wl.out_stride), dtype=synth.act_dtype(wl), device=dev)
        for i in range(10):
            elf.emb_dot_fwd(tab, batches[i % 2][0], batches[i % 2][1], out, None)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for i, (e0, e1) in enumerate(ev):
            e0.record()
            elf.emb_dot_fwd(tab, batches[i % 2][0], batches[i % 2][1], out, None)
            e1.record()
        torch.cuda.synchronize()
        lat = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        print(json.dumps({"metric": f"forward latency and samples/s, {wl.name}", "batch": B,
                          "mean_ms": round(float(lat.mean()), 4), "p50_ms": round(pct(lat, 50), 4),
                          "p90_ms": round(pct(lat, 90), 4), "p95_ms": round(pct(lat, 95), 4),
                          "p99_ms": round(pct(lat, 99), 4),
                          "samples_per_s": round(B / (float(lat.mean()) * 1e-3), 1),
                          "iters": iters, "data": "synthetic"}), flush=True)
        del batches, out
        torch.cuda.empty_cache()


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(wl, W, ro, batch, seconds):
    """The CPU oracle over batch 0 (same tables): the full batch when one run takes at most
    `seconds`, else its first `n` samples sized for `seconds`; three repetitions (median) when
    a run takes at most 10 s, else one.  samples/s on one host core (the process is pinned to
    one core while the oracle runs)."""
    from oracle import oracle as orc
    from tests.helpers import compact_tables, sub_batch, to_np

    bags, x0, G, idx, off = batch
    idx_h, off_h = to_np(idx), to_np(off)
    x0_h, G_h = to_np(x0), to_np(G)
    F, B, D = wl.num_tables, wl.batch, wl.dim
    table_bytes = W.numel() * W.element_size()
    full_tables = table_bytes <= (4 << 30)
    if full_tables:
        W_h, ro_h = to_np(W), to_np(ro)

    def run(n):
        samples = np.arange(n)
        si, so, nb = sub_batch(idx_h, off_h, F, B, samples)
        if full_tables:
            Wn, ron = W_h, ro_h
        else:  # only the rows the sample looks up (kept in row order)
            Wn, ron, si, _ = compact_tables(W, to_np(ro), si, so, F, nb)
        t = time.perf_counter()
        emb = orc.emb_bag_fwd(Wn, wl.table_dtype, ron, si, so, nb, D, wl.act_dtype)
        orc.dot_interact_fwd(x0_h[:n], emb, wl.act_dtype, wl.act_dtype, wl.out_stride)
        if wl.backward:
            _, demb = orc.dot_interact_bwd(x0_h[:n], emb, wl.act_dtype, G_h[:n], wl.act_dtype, wl.act_dtype)
            orc.grad_reduce_update(Wn, wl.table_dtype, ron, si, so, nb, demb, wl.act_dtype, wl.lr)
        return time.perf_counter() - t

    model, nproc = cpu_info()
    old = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(old)})
    try:
        # two probes separate the per-sample cost from the fixed one (the full-table SGD copy)
        n1, n2 = min(256, B), min(1024, B)
        t1 = run(n1)
        t2 = run(n2) if n2 > n1 else t1
        per_sample = max((t2 - t1) / max(n2 - n1, 1), t2 / max(n2, 1) * 0.5, 1e-9)
        fixed = max(t1 - per_sample * n1, 0.0)
        full_s = fixed + per_sample * B
        n = B if full_s <= seconds else int(min(B, max(n2, (seconds - fixed) / per_sample)))
        est = fixed + per_sample * n
        reps = 3 if est <= 10.0 else 1
        dts = [run(n) for _ in range(reps)]
        dt = float(np.median(dts))
    finally:
        os.sched_setaffinity(0, old)
    # the same oracle source built with OpenMP (bags / samples over all host threads; the
    # update stays serial), on the same sample
    from oracle import build as obuild
    omp = None
    if os.path.exists(obuild.LIB_OMP):
        prev = orc.use_library(obuild.LIB_OMP)
        try:
            dt_omp = float(np.median([run(n) for _ in range(3)]))
        finally:
            orc.restore_library(prev)
        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(old)
        omp = {"value": round(n / dt_omp, 1), "unit": "samples/s", "cores": threads,
               "kind": "oracle, OpenMP build (forward and interaction backward threaded)",
               "sample": f"the same {n} samples, median of 3 repetitions of {dt_omp:.1f} s"}
    tables = "full tables" + ("; full-table SGD copy" if wl.backward else "") if full_tables \
        else "only the looked-up rows of the tables"
    why = "" if n == B else (f"; not the full batch: one full-batch run would take about "
                             f"{full_s:.0f} s single-threaded, beyond the {seconds:.0f} s this leg is given")
    what = f"all {B} samples" if n == B else f"first {n} of {B} samples"
    runs = f"median of {reps} repetitions of {dt:.1f} s" if reps > 1 else \
        f"one run of {dt:.1f} s (a run above 10 s is not repeated)"
    res = {"value": round(n / dt, 1), "unit": "samples/s", "cores": 1, "kind": "oracle",
           "sample": f"{what} of batch 0 (all {F} tables, {tables}), "
                     f"single-threaded C oracle pinned to one core, {runs}{why}",
           "host_cpu": model, "host_cpus_visible": nproc}
    return res, omp


if __name__ == "__main__":
    main()
