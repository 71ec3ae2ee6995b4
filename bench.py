"""Throughput of the embedding-bag + dot-interaction training step on one MI355X.

One step = the whole hot path over one batch of synthetic input already resident in HBM:
  emb_bag_fwd -> dot_interact_fwd -> dot_interact_bwd -> emb_grad_reduce_update
on the train_step workload (B = 65536, 26 fp32 tables x 100,000 x 128, bf16 activations,
Zipf(1.05) hotness-1 indices, SGD lr 0.01).  Eight distinct index batches rotate across
steps so that no step replays the previous one's rows from cache.

Prints one JSON line: samples/s, the step time, the roofline of the dominant kernel
(algorithmic bytes / its HIP-event time vs the 8 TB/s HBM peak) and the CPU oracle
timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBPS = 8000.0
METRIC = "samples/s fwd+bwd (emb-bag + dot interaction) at batch 65536; achieved HBM GB/s"


def algorithmic_bytes(wl, nnz):
    """Bytes each call must move at minimum (every lookup's row counted; caches may serve
    part of them), per launch."""
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
        # dout in, x0 + emb in, dx0 + demb out
        "dot_interact_bwd": B * S * sa + 2 * B * V * D * sa,
        # sort: 3 LSD passes of key+value read/write; gradients gathered once; rows read+written
        "emb_grad_reduce_update": None,  # filled in by the caller (needs the unique-row count)
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="train_step")
    ap.add_argument("--batches", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB once (a plain copy kernel "
                         "of known size, to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import embedding_lookup_feature_amd as elf
    from embedding_lookup_feature_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = "cuda:0"
    torch.cuda.set_device(0)
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
    dx0 = torch.empty((B, D), dtype=act, device=dev)
    demb = torch.empty((B, F, D), dtype=act, device=dev)
    ws = torch.empty(max(elf.emb_grad_workspace_bytes(tab, b[0]) for b in batches), dtype=torch.uint8, device=dev)

    names = ["emb_bag_fwd", "dot_interact_fwd", "dot_interact_bwd", "emb_grad_reduce_update"]

    def step(i, ev=None):
        bags, x0, G = batches[i % len(batches)][:3]
        if ev: ev[0].record()
        elf.emb_bag_fwd(tab, bags, emb)
        if ev: ev[1].record()
        elf.dot_interact_fwd(x0, emb, out)
        if ev: ev[2].record()
        elf.dot_interact_bwd(x0, emb, G, dx0, demb)
        if ev: ev[3].record()
        elf.emb_grad_reduce_update(tab, bags, demb, wl.lr, ws)
        if ev: ev[4].record()

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps, no per-call events (nothing but the path in the stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # per-call durations: HIP events around each call, over the same number of steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    call_ms = {n: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs])) for k, n in enumerate(names)}

    nnz = batches[0][3].numel()
    algo = algorithmic_bytes(wl, nnz)
    idx0, off0 = batches[0][3], batches[0][4]
    # unique rows touched (for the update's row read + write), from the input indices
    keys = idx0.long() + torch.repeat_interleave(ro[:-1], (off0[1:].long() - off0[:-1].long()).view(F, B).sum(1))
    U = int(torch.unique(keys).numel())
    st = 4 if wl.table_dtype == "f32" else 2
    sa = 4 if wl.act_dtype == "f32" else 2
    algo["emb_grad_reduce_update"] = 8 * nnz + nnz * D * sa + 2 * U * D * st
    calls = {n: {"ms": round(call_ms[n], 4), "algo_bytes": int(algo[n]),
                 "algo_gbps": round(algo[n] / (call_ms[n] * 1e-3) / 1e9, 1)} for n in names}
    step_bytes = sum(algo.values())
    # dominant single-kernel call: the one with the longest time among the one-launch calls
    single = ["emb_bag_fwd", "dot_interact_fwd", "dot_interact_bwd"]
    dom = max(single, key=lambda n: call_ms[n])
    kernel = {"emb_bag_fwd": "k_emb_bag_fwd", "dot_interact_fwd": "k_dot_fwd_mfma",
              "dot_interact_bwd": "k_dot_bwd_mfma"}[dom]
    achieved = algo[dom] / (call_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}

    result = {
        "metric": METRIC,
        "value": round(B / (ms_per_step * 1e-3), 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.description}", "global_batch": B,
                   "tables": F, "rows_per_table": wl.rows[0], "dim": D,
                   "table_dtype": wl.table_dtype, "act_dtype": wl.act_dtype, "nnz": int(nnz),
                   "unique_rows": U, "parallelism": "single-gpu"},
        "hbm_gbps_algorithmic": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "calls": calls,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, W, ro, batches[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(wl, W, ro, batch, seconds):
    """The CPU oracle over the first `n` samples of batch 0 (same tables), sized so that
    the run takes about `seconds`; samples/s on one host core."""
    from oracle import oracle as orc
    from tests.helpers import sub_batch, to_np

    bags, x0, G, idx, off = batch
    W_h, ro_h, idx_h, off_h = to_np(W), to_np(ro), to_np(idx), to_np(off)
    x0_h, G_h = to_np(x0), to_np(G)
    F, B, D = wl.num_tables, wl.batch, wl.dim

    def run(n):
        samples = np.arange(n)
        si, so, nb = sub_batch(idx_h, off_h, F, B, samples)
        t = time.perf_counter()
        emb = orc.emb_bag_fwd(W_h, wl.table_dtype, ro_h, si, so, nb, D, wl.act_dtype)
        orc.dot_interact_fwd(x0_h[:n], emb, wl.act_dtype, wl.act_dtype, wl.out_stride)
        _, demb = orc.dot_interact_bwd(x0_h[:n], emb, wl.act_dtype, G_h[:n], wl.act_dtype, wl.act_dtype)
        orc.grad_reduce_update(W_h, wl.table_dtype, ro_h, si, so, nb, demb, wl.act_dtype, wl.lr)
        return time.perf_counter() - t

    probe_n = 256
    dt = run(probe_n)
    n = int(min(B, max(probe_n, probe_n * seconds / max(dt, 1e-6))))
    dt = run(n)
    return {"value": round(n / dt, 1), "unit": "samples/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {B} samples of batch 0 (all {F} tables; full-table SGD copy), "
                      f"single-threaded C oracle, {dt:.1f} s"}


if __name__ == "__main__":
    main()
